// dwc_mfma_batch16.h -- packed-MFMA forward-type kernel of libdwc with 16
// images in the matrix rows and two channels per wave (bf16/fp16 operands,
// gfx950 v_mfma_f32_16x16x32_{bf16,f16}, fp32 accumulation).
//
// The same packing as fwd_mfma_batch (Flash-DWC §4.2, Fig. 8, with the
// batch as the second matrix dimension): for one output row oh, one filter
// row fh and the input row r = oh + fh - PH,
//   A[i][k] = x[n0 + i][r][k]                        (16 images x 32 input columns)
//   B[k][j] = w[fh][k - (16 g + j) + PW]  (0 <= . < FW, else 0)   (32 x 16 output columns)
//   D[i][j] += sum_k A[i][k] B[k][j]
// accumulates output column 16 g + j of row oh for 16 images; NG = 1 or 2
// column groups cover output widths up to 16 or 32.  K = 32 covers the
// whole input row (widths up to 32), so one A per staged row and channel.
//
// Why 16 images and 16 channels per workgroup instead of 32 x 8: a
// workgroup's global loads and stores touch one 128-byte line per pixel
// whatever part of it they use.  With 16 channels (32 bytes of a pixel)
// the loads and stores of one output row touch half as many lines as with
// 8 channels, at the same register cost: a wave holds two channels' 16
// images where the 32-image kernel holds one channel's 32.
//
// A workgroup owns 16 channels (two per wave) x 16 images x R output rows;
// the R rows at filter row fh read stream rows fh .. fh + R - 1, so each
// channel keeps a ring of R A registers that takes one new row per filter
// row (nothing moves between lanes), and the band B of (channel, fh, g) is
// read once per filter row and serves all R output rows.
//
// Operand staging (LDS):
//   * input rows stream through kB16Slots row slots, two rows per barrier,
//     the next two rows' global loads in flight during the current rows'
//     MFMAs.  A slot holds, per channel and 8-column group q, the 16
//     images' 8 columns: lane (q, i) of the A read takes 16 contiguous
//     bytes.  Thread (image, column pair p, channel half h) loads the two
//     pixels' 8 channels (16 bytes each; the two halves of a pixel are
//     neighbouring lanes, one 32-byte piece of the line) and writes 8
//     dwords of column pairs.  The pitches put the 64 dword writes of one
//     instruction on 64 different banks;
//   * the filter band, as in fwd_mfma_batch: per channel and filter row, 32
//     zeros, the FW taps (turned by 180 degrees for FLIP) and 32 - FW zeros;
//     the next row's leading zeros end the row.  Lane (q, j) of column
//     group g needs elements e = 32 + 8 q - 16 g - j + PW .. e + 7, read as
//     5 aligned dwords and shifted by v_alignbit;
//   * outputs pass through LDS, as many rows at a time as the LDS holds, so
//     that global stores are 16-byte writes of 64-byte pixel pieces.
// Zero padding: staged columns and images past the input read 0 through
// the buffer resource's range check; padding rows are never staged nor
// multiplied.
#pragma once

#include <type_traits>

#include "dwc_device.h"
#include "dwc_mfma.h"
#include "dwc_mfma8.h"

namespace dwc {

typedef uint32_t b16_u32x2 __attribute__((ext_vector_type(2)));

// One lane's matrix operand: 8 elements, 16 bytes (bf16 / fp16) or 8 bytes
// (fp8), and the 16x16x32 MFMA that takes it.
template <int DT>
struct B16Op {
  static constexpr bool b8 = DT == DT_E4M3 || DT == DT_E5M2;
  typedef typename std::conditional<b8, b16_u32x2, mf_u32x4>::type T;
};

template <int DT>
__device__ __forceinline__ mf_f32x4 mfma_b16(typename B16Op<DT>::T a, typename B16Op<DT>::T b,
                                             mf_f32x4 c) {
  if constexpr (DT == DT_E4M3)
    return __builtin_amdgcn_mfma_f32_16x16x32_fp8_fp8(__builtin_bit_cast(long, a),
                                                      __builtin_bit_cast(long, b), c, 0, 0, 0);
  else if constexpr (DT == DT_E5M2)
    return __builtin_amdgcn_mfma_f32_16x16x32_bf8_bf8(__builtin_bit_cast(long, a),
                                                      __builtin_bit_cast(long, b), c, 0, 0, 0);
  else
    return mfma_16x16x32<DT>(a, b, c);
}

// DPP quad_perm [1, 0, 3, 2]: each lane takes its neighbour's value (lane
// pairs 2k, 2k + 1 swap).
__device__ __forceinline__ uint32_t swap_pair(uint32_t v) {
  return (uint32_t)__builtin_amdgcn_mov_dpp((int)v, 0xB1, 0xF, 0xF, false);
}

template <int DT, int NG, bool FLIP>
__global__ __launch_bounds__(512, 1) void fwd_mfma_batch16(MfmaBatchArgs a) {
  extern __shared__ __align__(16) unsigned char lds[];
  typedef typename B16Op<DT>::T Op;
  constexpr bool B8 = B16Op<DT>::b8;
  constexpr int EB = B8 ? 1 : 2;                // bytes per element
  constexpr int NT = 512;
  constexpr int CB = kB16Cb;                   // 16 channels, two per wave
  constexpr int R = kB16Rows;
  constexpr int ZROW = 64 * EB;                 // band bytes per filter row (64 elements)
  constexpr int KQP = B8 ? kB16KqPitch8 : kB16KqPitch;  // bytes per (channel, 8-column group)
  constexpr int CHP = B8 ? kB16ChPitch8 : kB16ChPitch;  // bytes per channel in a staged row
  constexpr int SLOT = CB * CHP;                // bytes per staged input row
  constexpr int OPITCH = kB16Opitch;            // floats per staged output pixel
  const int tid = threadIdx.x;
  const int wave = uniform(tid >> 6);
  const int lane = tid & 63;
  const int blk = xcd_logical_block(blockIdx.x, gridDim.x);
  if (blk >= a.num_blocks) return;  // the whole workgroup leaves together
  // Workgroup (channel block, row chunk, image group); logical ids run over
  // groups of gw channel blocks first (whole lines of each pixel), then row
  // chunks, so that the workgroups an XCD holds at once read the same input
  // rows and write whole output lines.
  int t = blk;
  const int gw = a.cblk % (64 / CB) == 0 ? 64 / CB : 1;
  const int cbg = t % gw;
  t /= gw;
  const int rc = t % a.rch;
  t /= a.rch;
  const int ncg = a.cblk / gw;
  const int cbk = (t % ncg) * gw + cbg;
  const int ig = t / ncg;
  const int n0 = ig * kB16Img;
  const int c0 = cbk * CB, oh0 = rc * R;
  const int FH = a.FH, FW = a.FW;
  const int zrows = FH + 1;                     // one zero row after the last
  unsigned char* zt = lds;                      // [CB ch][FH + 1][ZROW bytes]
  unsigned char* ring = lds + CB * zrows * ZROW;  // kB16Slots staged rows

  // ---- staging of input rows.  One buffer resource over the image group
  // (wave-uniform); an item's image is part of its offset, and images past
  // N fall outside the range.  Staged element (ch, col = 8 q + e, image i)
  // sits at byte ch * CHP + q * KQP + (8 i + e) * EB.
  //   bf16 / fp16: thread (image si, column pair sp, channel half sh),
  //     tid = (si * 16 + sp) * 2 + sh, loads both pixels' 8 channels and
  //     writes the dword of columns (2 sp, 2 sp + 1) of each of them; both
  //     rows of a batch are loaded by every thread.
  //   fp8: thread (row su of the batch, image si, column pair sp), tid =
  //     ((su * 16 + si) * 16 + sp), loads both pixels' 16 channels; lane
  //     pairs trade half their channels (DPP), so that each lane holds 4
  //     columns of 8 channels (sh = sp & 1: channels 8 sh .. 8 sh + 7) and
  //     writes their dwords after a 4x4 byte transpose.
  const uint32_t Cb = (uint32_t)a.C * EB;
  const uint32_t img_bytes = (uint32_t)(a.IH * a.IW) * Cb;
  const int su = B8 ? tid >> 8 : 0;
  const int sh = B8 ? (tid & 1) : (tid & 1);
  const int sp = B8 ? (tid & 15) : ((tid >> 1) & 15);
  const int si = B8 ? ((tid >> 4) & 15) : (tid >> 5);
  const int scol = 2 * sp;
  const bool ok0 = scol < a.IW, ok1 = scol + 1 < a.IW;
  const uint32_t scoff =
      (uint32_t)si * img_bytes +
      ((uint32_t)scol * (uint32_t)a.C + (uint32_t)(c0 + (B8 ? 0 : 8 * sh))) * EB;
  const int s_dst = B8 ? 8 * sh * CHP + (sp >> 2) * KQP + si * 8 + ((sp >> 1) & 1) * 4
                       : 8 * sh * CHP + (sp >> 2) * KQP + si * 16 + (sp & 3) * 4;
  const int r_base = oh0 - a.PH;  // image row of stream row q = 0
  auto row_ok = [&](int q) { return q < a.nq && (unsigned)(r_base + q) < (unsigned)a.IH; };
  const auto rs = make_rsrc((const char*)a.in + (size_t)n0 * img_bytes,
                            (uint32_t)min(kB16Img, a.N - n0) * img_bytes);
  struct Stage {
    mf_u32x4 v0, v1;
  };
  // u: the row's place in its batch of two (fp8: the half of the threads
  // that stages it)
  auto stage_load = [&](int q, int u, Stage& st) {
    if (B8 && su != u) return;  // wave-uniform
    const bool rok = row_ok(q);
    const uint32_t o = (uint32_t)(r_base + q) * (uint32_t)a.IW * Cb + scoff;
    st.v0 = __builtin_bit_cast(
        mf_u32x4, __builtin_amdgcn_raw_buffer_load_b128(rs, (int)(rok && ok0 ? o : kOOB), 0, 0));
    st.v1 = __builtin_bit_cast(
        mf_u32x4,
        __builtin_amdgcn_raw_buffer_load_b128(rs, (int)(rok && ok1 ? o + Cb : kOOB), 0, 0));
  };
  auto stage_store = [&](int q, int u, const Stage& st) {
    if (B8 && su != u) return;  // wave-uniform
    if (!row_ok(q)) return;     // a padding row is never read
    unsigned char* d = ring + (q % kB16Slots) * SLOT + s_dst;
    if constexpr (B8) {
      // the even lane keeps channels 0-7 and sends 8-15, the odd lane the
      // reverse; columns of the quad: even lane own 0, 1 and received 2, 3,
      // odd lane received 0, 1 and own 2, 3
      uint32_t c[4][2];
#pragma unroll
      for (int w = 0; w < 2; ++w) {
        const uint32_t r0 = swap_pair(sh ? st.v0[w] : st.v0[w + 2]);
        const uint32_t r1 = swap_pair(sh ? st.v1[w] : st.v1[w + 2]);
        const uint32_t o0 = sh ? st.v0[w + 2] : st.v0[w];
        const uint32_t o1 = sh ? st.v1[w + 2] : st.v1[w];
        c[0][w] = sh ? r0 : o0;
        c[1][w] = sh ? r1 : o1;
        c[2][w] = sh ? o0 : r0;
        c[3][w] = sh ? o1 : r1;
      }
#pragma unroll
      for (int w = 0; w < 2; ++w) {
        uint32_t ch[4];
        transpose4(c[0][w], c[1][w], c[2][w], c[3][w], ch);
#pragma unroll
        for (int i = 0; i < 4; ++i) *(uint32_t*)(d + (4 * w + i) * CHP) = ch[i];
      }
    } else {
#pragma unroll
      for (int j = 0; j < 8; ++j, d += CHP)
        *(uint32_t*)d = __builtin_amdgcn_perm(st.v1[j >> 1], st.v0[j >> 1],
                                              (j & 1) ? 0x07060302u : 0x05040100u);
    }
  };

  // ---- start-up: the first two stream rows' loads and the filter taps'
  // loads go out first, so that their latency overlaps the band's zero fill.
  const int q_lo = max(0, a.PH - oh0);
  constexpr int PD = kB16Prefetch;
  Stage pf[PD][2];
#pragma unroll
  for (int k = 0; k < PD; ++k) {
    stage_load(q_lo + 2 * k, 0, pf[k][0]);
    stage_load(q_lo + 2 * k + 1, 1, pf[k][1]);
  }
  // filter band: per channel and filter row, 32 zeros, the taps, zeros up
  // to the next row.  Items: bf16 / fp16 (tap, channel half), te = 2 tap +
  // half; fp8 one tap (16 channels) each; item te on thread te % NT.
  constexpr int TPI = B8 ? 1 : 2;               // items per tap
  const int ftaps = FH * FW;
  const int titems = uniform((TPI * ftaps + NT - 1) / NT);  // <= kB16TapItems
  mf_u32x4 tv[kB16TapItems];
  {
    const auto frsrc = make_rsrc(a.filt, (uint32_t)ftaps * (uint32_t)a.C * EB);
#pragma unroll
    for (int k = 0; k < kB16TapItems; ++k) {
      if (k >= titems) break;                   // uniform
      const int te = tid + k * NT;
      const int hf = B8 ? 0 : te & 1, tap = B8 ? te : te >> 1;
      const int src = FLIP ? ftaps - 1 - tap : tap;
      const uint32_t off = te < TPI * ftaps
                               ? ((uint32_t)src * (uint32_t)a.C + (uint32_t)(c0 + 8 * hf)) * EB
                               : kOOB;
      tv[k] = __builtin_bit_cast(mf_u32x4,
                                 __builtin_amdgcn_raw_buffer_load_b128(frsrc, (int)off, 0, 0));
    }
  }
  const int zlen16 = CB * zrows * ZROW / 16;
  for (int i = tid; i < zlen16; i += NT) ((mf_u32x4*)zt)[i] = mf_u32x4{0u, 0u, 0u, 0u};
  __syncthreads();
#pragma unroll
  for (int k = 0; k < kB16TapItems; ++k) {
    if (k >= titems) break;                     // uniform
    const int te = tid + k * NT;
    if (te < TPI * ftaps) {
      const int hf = B8 ? 0 : te & 1, tap = B8 ? te : te >> 1;
      const int fh = fast_div(tap, a.fw_magic), fw = tap - fh * FW;
      unsigned char* d = zt + (8 * hf * zrows + fh) * ZROW + (32 + fw) * EB;
      if constexpr (B8) {
#pragma unroll
        for (int j = 0; j < 16; ++j, d += zrows * ZROW)
          *d = (unsigned char)(tv[k][j >> 2] >> (8 * (j & 3)));
      } else {
#pragma unroll
        for (int j = 0; j < 8; ++j, d += zrows * ZROW)
          *(uint16_t*)d = (uint16_t)((tv[k][j >> 1] >> (16 * (j & 1))) & 0xffffu);
      }
    }
  }

  // ---- compute operands.  A: lane (q, i) reads the 8 elements of image
  // i, column group q of a staged row.  B: lane (q, j) of column group g
  // starts at element e = 32 + 8 q - 16 g - j + PW of its channel's band
  // row: 5 (3) aligned dwords from the one at or below, shifted by
  // v_alignbit (v_alignbyte).  D: lane (q, j) holds images 4 q .. 4 q + 3
  // at column 16 g + j.
  const int lq = lane >> 4, lm = lane & 15;
  const int a_lane = 2 * wave * CHP + lq * KQP + lm * 8 * EB;
  auto read_a = [&](int q, int cc) -> Op {
    return *(const Op*)(ring + (q % kB16Slots) * SLOT + a_lane + cc * CHP);
  };
  const int e0 = 32 + 8 * lq - lm + a.PW;        // element of column group 0
  const uint32_t* zrow0 =
      (const uint32_t*)(zt + 2 * wave * zrows * ZROW + ((e0 * EB) & ~3));
  const uint32_t bsel = B8 ? (uint32_t)(e0 & 3) : (uint32_t)(e0 & 1) * 16u;
  auto read_b = [&](int cc, int fh, int g) -> Op {
    const uint32_t* p = zrow0 + (cc * zrows + fh) * (ZROW / 4) - 4 * EB * g;
    if constexpr (B8) {
      const uint32_t d0 = p[0], d1 = p[1], d2 = p[2];
      return Op{__builtin_amdgcn_alignbyte(d1, d0, bsel), __builtin_amdgcn_alignbyte(d2, d1, bsel)};
    } else {
      mf_u32x4 d;
      __builtin_memcpy(&d, p, 16);
      const uint32_t d4 = p[4];
      return mf_u32x4{__builtin_amdgcn_alignbit(d[1], d[0], bsel),
                      __builtin_amdgcn_alignbit(d[2], d[1], bsel),
                      __builtin_amdgcn_alignbit(d[3], d[2], bsel),
                      __builtin_amdgcn_alignbit(d4, d[3], bsel)};
    }
  };

  // Stream rows q = 0 .. nq - 1 (nq = R + FH - 1); row q completes the
  // operands of filter row fh = q - R + 1.  Only rows q_lo .. q_hi - 1 are
  // image rows; the stream runs from q_lo (earlier rows are padding, whose
  // products are never formed) to q_hi + R - 1 (later filter rows read
  // padding rows only), so that a workgroup whose window hangs over the
  // image spends no barriers on padding.  Row q sits in LDS slot
  // q % kB16Slots and in ring register (q - q_lo) % R.
  const int q_hi = min(a.nq, a.IH + a.PH - oh0);
  const int nloc = max(0, min(a.nq, q_hi + R - 1) - q_lo);  // rows streamed
  // band of the next filter row, read during the current row's MFMAs (the
  // band does not change, so this read may cross a barrier); rows clamp to
  // [0, FH - 1] where no filter row follows.  The first read waits for
  // every wave's tap writes.
  auto fh_clamp = [&](int fh) { return min(max(fh, 0), FH - 1); };
  __syncthreads();
  Op bn[2][NG];
#pragma unroll
  for (int cc = 0; cc < 2; ++cc)
#pragma unroll
    for (int g = 0; g < NG; ++g) bn[cc][g] = read_b(cc, fh_clamp(q_lo - (R - 1)), g);
  mf_f32x4 acc[2][R][NG];
#pragma unroll
  for (int cc = 0; cc < 2; ++cc)
#pragma unroll
    for (int j = 0; j < R; ++j)
#pragma unroll
      for (int g = 0; g < NG; ++g) acc[cc][j][g] = mf_f32x4{0.f, 0.f, 0.f, 0.f};
  Op ringA[2][R];  // stream row q of channel cc in ringA[cc][(q - q_lo) % R]

  // Rows 2 b, 2 b + 1 (from q_lo) go to LDS at barrier b while rows
  // 2 (b + PD), 2 (b + PD) + 1 are loaded.  The loop body covers 2 PD R
  // rows, so that ring and prefetch indices are compile-time.
  for (int l0 = 0; l0 < nloc; l0 += 2 * PD * R) {
#pragma unroll
    for (int bq = 0; bq < PD * R; ++bq) {
      const int la = l0 + 2 * bq;
      if (la >= nloc) break;                  // uniform
      const int qa = q_lo + la;
      const int k = bq % PD;                  // l0 is a multiple of 2 PD
      // slots of rows qa, qa + 1 were last read before the previous barrier
      stage_store(qa, 0, pf[k][0]);
      stage_store(qa + 1, 1, pf[k][1]);
      stage_load(qa + 2 * PD, 0, pf[k][0]);
      stage_load(qa + 2 * PD + 1, 1, pf[k][1]);
      __syncthreads();
#pragma unroll
      for (int u = 0; u < 2; ++u) {
        const int q = qa + u;
        const int slot = (2 * bq + u) % R;    // (q - q_lo) % R: l0 is a multiple of R
        if (la + u >= nloc) break;
        if (row_ok(q)) {
          ringA[0][slot] = read_a(q, 0);
          ringA[1][slot] = read_a(q, 1);
        }
        const int fh = q - (R - 1);
        Op b[2][NG];
#pragma unroll
        for (int cc = 0; cc < 2; ++cc)
#pragma unroll
          for (int g = 0; g < NG; ++g) {
            b[cc][g] = bn[cc][g];
            bn[cc][g] = read_b(cc, fh_clamp(fh + 1), g);
          }
        if (fh < 0) continue;                 // still filling the ring
#pragma unroll
        for (int j = 0; j < R; ++j) {
          // output row oh0 + j reads stream row fh + j = q - (R - 1) + j,
          // which is an image row only from q_lo on (so its ring register
          // has been written)
          const int r = r_base + fh + j;
          if ((unsigned)r >= (unsigned)a.IH || oh0 + j >= a.OH) continue;  // uniform
          const int s = (2 * bq + u + 1 + j) % R;  // (q - q_lo - R + 1 + j) % R
#pragma unroll
          for (int cc = 0; cc < 2; ++cc)
#pragma unroll
            for (int g = 0; g < NG; ++g)
              acc[cc][j][g] = mfma_b16<DT>(ringA[cc][s], b[cc][g], acc[cc][j][g]);
        }
      }
    }
  }

  // ---- outputs: registers -> LDS [image][column][channel] -> 16-byte
  // stores of 4 channels, a.orows output rows per pair of barriers.  Lane
  // (q, j), register v of (channel cc, group g) holds image 4 q + v at
  // column 16 g + j; the wave's two channels are neighbouring floats.
  const int oimgs = min(kB16Img, a.N - n0);
  const int ipitch = a.OW * OPITCH + 4;        // floats per staged image
  const int row_floats = kB16Img * ipitch;
  float* const ostage = (float*)lds;
  float* const obase = a.out + ((size_t)n0 * a.OH + oh0) * a.OW * a.C + c0;
  const uint32_t row_step = (uint32_t)a.OW * (uint32_t)a.C;  // floats per output row
  const int nitems = kB16Img * a.OW * 4;       // (pixel, channel quad) items per row
  auto stage_row = [&](int j, float* dst) {
#pragma unroll
    for (int g = 0; g < NG; ++g) {
      const int col = 16 * g + lm;
      if (col < a.OW) {
#pragma unroll
        for (int v = 0; v < 4; ++v) {
          float* d = dst + (4 * lq + v) * ipitch + col * OPITCH + 2 * wave;
          *(float2*)d = float2{acc[0][j][g][v], acc[1][j][g][v]};
        }
      }
    }
  };
  auto store_row = [&](int j, const float* src) {
    for (int it = tid; it < nitems; it += NT) {
      const int qd = it & 3, pc = it >> 2;
      const int img = fast_div(pc, a.ow_magic), col = pc - img * a.OW;
      if (img >= oimgs) break;                 // items run image by image
      const mf_f32x4 v = *(const mf_f32x4*)(src + img * ipitch + col * OPITCH + 4 * qd);
      const uint32_t og = ((uint32_t)img * (uint32_t)a.OH * (uint32_t)a.OW + (uint32_t)col) *
                              (uint32_t)a.C + 4u * (uint32_t)qd;
      *(mf_f32x4*)(obase + (og + (uint32_t)j * row_step)) = v;
    }
  };
  int nb = 0;  // rows staged in the current round
#pragma unroll
  for (int j = 0; j < R; ++j) {
    if (oh0 + j >= a.OH) break;               // uniform
    if (nb == 0) __syncthreads();             // the staging area is free
    stage_row(j, ostage + nb * row_floats);
    ++nb;
    if (nb == a.orows || j + 1 == R || oh0 + j + 1 >= a.OH) {
      __syncthreads();
      for (int k = 0; k < nb; ++k) store_row(j + 1 - nb + k, ostage + k * row_floats);
      nb = 0;
    }
  }
}

}  // namespace dwc
