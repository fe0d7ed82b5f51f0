// dwc_mfma_batch.h -- packed-MFMA forward-type kernel of libdwc with the
// batch in the matrix rows, 32-image form (bf16/fp16 operands, gfx950
// v_mfma_f32_32x32x16_{bf16,f16}, fp32 accumulation).  The planner takes it
// where the 16-image form (dwc_mfma_batch16.h: half the cache lines per
// staged row) does not apply, i.e. C % 16 != 0, or when asked for.
//
// The GEMV-to-GEMM packing of Flash-DWC (§4.2, Fig. 8) needs a second
// matrix dimension next to the filter's Toeplitz band.  Here that dimension
// is the batch: every image of a channel meets the same filter, so for one
// output row oh, one filter row fh and one 16-column chunk kc of the input
// row r = oh + fh - PH,
//   A[i][k] = x[n0 + i][r][16 kc + k]                 (32 images x 16 input columns)
//   B[k][j] = w[fh][16 kc + k - j + PW]  (0 <= . < FW, else 0)   (16 x 32 output columns)
//   D[i][j] += sum_k A[i][k] B[k][j]
// accumulates output column j of row oh for 32 images.  Compared with
// packing output rows into the matrix rows:
//   * K runs over the input's real columns only (IW <= 32: two chunks), so
//     no instruction multiplies the zero padding around the image, and
//     filter rows that fall on padding rows are skipped (a uniform branch);
//   * A of one input row serves every output row that reads it, and the
//     workgroup's output rows are consecutive, so the R rows a wave's
//     accumulators need at filter row fh are rows fh .. fh + R - 1 of a
//     stream: a ring of R registers per chunk takes one new row per filter
//     row and nothing moves between lanes;
//   * the band B of (fh, kc) is read once per filter row and serves the R
//     output rows of the wave.
// A workgroup owns 8 channels (one per wave) x 32 images x R output rows.
//
// Operand staging (LDS):
//   * input rows stream through a ring of kBatchSlots row slots, two rows
//     per barrier.  A slot holds, per channel, chunk and half (8 columns),
//     the 32 images' 8 columns: lane (i, h) of the A read takes 16
//     contiguous bytes.  Each thread loads two adjacent pixels (8 channels
//     each) of one image and writes the 8 channel pairs as dwords;
//   * the filter band: per channel and filter row, 32 zeros, the FW taps
//     (turned by 180 degrees for FLIP) and 32 - FW zeros; the next row's
//     leading zeros end the row.  Lane (j, h) of chunk kc needs elements
//     e = 16 kc + 8 h - j + PW + 32 .. e + 7, read as 5 aligned dwords and
//     shifted by v_alignbit (2-byte-aligned 16-byte reads run at a quarter
//     of the rate);
//   * outputs pass through LDS, one output row at a time, so that global
//     stores are channel-contiguous 16-byte writes.
// A workgroup computes one image group of 32 (a loop over several groups
// made the compiler keep per-group offsets live across the row loop and
// spill).  Its LDS (the band and four row slots: 92-104 KB from 17 to 31
// filter rows) and registers leave room for one workgroup per CU.
// Zero padding: staged columns and images past the input read 0 through
// the buffer resource's range check; padding rows are never staged nor
// multiplied.
#pragma once

#include <type_traits>

#include "dwc_device.h"
#include "dwc_mfma.h"

namespace dwc {

typedef __bf16 mb_bf16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 mb_f16x8 __attribute__((ext_vector_type(8)));
typedef float mb_f32x16 __attribute__((ext_vector_type(16)));

template <int DT>
__device__ __forceinline__ mb_f32x16 mfma_32x32x16(mf_u32x4 a, mf_u32x4 b, mb_f32x16 c) {
  if constexpr (DT == DT_BF16) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(mb_bf16x8, a),
                                                   __builtin_bit_cast(mb_bf16x8, b), c, 0, 0, 0);
  } else {
    return __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(mb_f16x8, a),
                                                  __builtin_bit_cast(mb_f16x8, b), c, 0, 0, 0);
  }
}

typedef uint32_t mb_u32x2 __attribute__((ext_vector_type(2)));

// CB channels of a pixel (CB / 2 dwords: 8 channels one 16-byte load, 4
// channels an 8-byte load) through a buffer resource.
template <int CB>
struct ChanVec {
  typedef typename std::conditional<CB == 8, mf_u32x4, mb_u32x2>::type T;
  __device__ static T load(__amdgpu_buffer_rsrc_t r, uint32_t off) {
    if constexpr (CB == 8)
      return __builtin_bit_cast(T, __builtin_amdgcn_raw_buffer_load_b128(r, (int)off, 0, 0));
    else
      return __builtin_bit_cast(T, __builtin_amdgcn_raw_buffer_load_b64(r, (int)off, 0, 0));
  }
};

// CB channels per workgroup (one per wave), CB = 8 or 4.
template <int DT, int CB, bool FLIP>
__global__ __launch_bounds__(64 * CB, 2) void fwd_mfma_batch(MfmaBatchArgs a) {
  extern __shared__ __align__(16) unsigned char lds[];
  constexpr int NT = 64 * CB;
  constexpr int IT = kBatchImg * 16 / NT;      // staging items (pixel pairs) per thread and row
  using CV = ChanVec<CB>;
  typedef typename CV::T PV;
  constexpr int R = kBatchRows;
  constexpr int ZROW = 64;                      // band elements per filter row
  constexpr int HP = kBatchHalfPitch;           // bytes per (channel, chunk, half) plane
  constexpr int SLOT = CB * 4 * HP;             // bytes per staged input row
  constexpr int OPITCH = CB == 8 ? 12 : 4;      // floats per staged output pixel
  const int tid = threadIdx.x;
  const int wave = uniform(tid >> 6);
  const int lane = tid & 63;
  const int blk = xcd_logical_block(blockIdx.x, gridDim.x);
  if (blk >= a.num_blocks) return;  // the whole workgroup leaves together
  // Workgroup (channel block, row chunk, image group).
  // Logical ids run over groups of gw channel blocks first, then row
  // chunks, so that the workgroups an XCD holds at once write whole lines
  // of each output pixel (gw blocks, 64 channels: 256 bytes) and read the
  // same input rows.
  int t = blk;
  const int gw = a.cblk % (64 / CB) == 0 ? 64 / CB : 1;
  const int cb8 = t % gw;
  t /= gw;
  const int rc = t % a.rch;
  t /= a.rch;
  const int ncg = a.cblk / gw;
  const int cbk = (t % ncg) * gw + cb8;
  const int ig = t / ncg;
  const int n0 = ig * kBatchImg;
  const int c0 = cbk * CB, oh0 = rc * R;
  const int FH = a.FH, FW = a.FW;
  const int zrows = FH + 1;                     // one zero row after the last
  uint16_t* zt = (uint16_t*)lds;                // [CB ch][FH + 1][ZROW]
  unsigned char* ring = lds + CB * zrows * ZROW * 2;  // kBatchSlots staged rows

  // ---- filter band: zero it, then write the taps after a barrier
  const int zlen8 = CB * zrows * ZROW / 8;
  for (int i = tid; i < zlen8; i += NT) ((mf_u32x4*)zt)[i] = mf_u32x4{0u, 0u, 0u, 0u};
  __syncthreads();
  {
    const auto frsrc = make_rsrc(a.filt, (uint32_t)(FH * FW) * (uint32_t)a.C * 2u);
    const int ftaps = FH * FW;
    for (int te = tid; te < ftaps; te += NT) {
      const int src = FLIP ? ftaps - 1 - te : te;
      const PV v = CV::load(frsrc, ((uint32_t)src * (uint32_t)a.C + (uint32_t)c0) * 2u);
      const int fh = fast_div(te, a.fw_magic), fw = te - fh * FW;
      uint16_t* d = zt + fh * ZROW + 32 + fw;
#pragma unroll
      for (int j = 0; j < CB; ++j, d += zrows * ZROW)
        *d = (uint16_t)((v[j >> 1] >> (16 * (j & 1))) & 0xffffu);
    }
  }

  // ---- staging of input rows: item (image si, column pair sp) of a row;
  // thread tid has items tid + k NT, k < IT.  One buffer resource over an
  // image group (wave-uniform); an item's image is part of its offset, and
  // images past N fall outside the range.
  const uint32_t Cb = (uint32_t)a.C * 2u;
  const int sp = tid & 15;
  const uint32_t img_bytes = (uint32_t)(a.IH * a.IW) * Cb;
  const int scol = 2 * sp;
  const bool ok0 = scol < a.IW, ok1 = scol + 1 < a.IW;
  const uint32_t scoff =
      (uint32_t)(tid >> 4) * img_bytes + ((uint32_t)scol * (uint32_t)a.C + (uint32_t)c0) * 2u;
  constexpr int IMG_STEP = NT / 16;  // images from one item of a thread to the next
  // staged element (ch, col = 16 kc + 8 h + e, image i) sits at byte
  // ch * 4 HP + (2 kc + h) * HP + (i * 8 + e) * 2; an item writes the dword
  // of columns (scol, scol + 1) for each of its CB channels
  const int s_dst = ((sp >> 2) * HP) + ((tid >> 4) * 8 + 2 * (sp & 3)) * 2;
  const int r_base = oh0 - a.PH;  // image row of stream row q = 0
  auto row_ok = [&](int q) { return q < a.nq && (unsigned)(r_base + q) < (unsigned)a.IH; };
  const auto rs = make_rsrc((const char*)a.in + (size_t)n0 * img_bytes,
                            (uint32_t)min(kBatchImg, a.N - n0) * img_bytes);
  struct Stage {
    PV v0[IT], v1[IT];
  };
  auto stage_load = [&](__amdgpu_buffer_rsrc_t rs, int q, Stage& st) {
    const bool rok = row_ok(q);
    const uint32_t off = (uint32_t)(r_base + q) * (uint32_t)a.IW * Cb + scoff;
#pragma unroll
    for (int k = 0; k < IT; ++k) {
      const uint32_t o = off + (uint32_t)(k * IMG_STEP) * img_bytes;
      st.v0[k] = CV::load(rs, rok && ok0 ? o : kOOB);
      st.v1[k] = CV::load(rs, rok && ok1 ? o + Cb : kOOB);
    }
  };
  auto stage_store = [&](int q, const Stage& st) {
    if (!row_ok(q)) return;  // a padding row is never read
#pragma unroll
    for (int k = 0; k < IT; ++k) {
      unsigned char* d = ring + (q % kBatchSlots) * SLOT + s_dst + k * IMG_STEP * 16;
#pragma unroll
      for (int j = 0; j < CB; ++j, d += 4 * HP)
        *(uint32_t*)d = __builtin_amdgcn_perm(st.v1[k][j >> 1], st.v0[k][j >> 1],
                                              (j & 1) ? 0x07060302u : 0x05040100u);
    }
  };

  // ---- compute operands.  A: lane (i, h) reads the 16 bytes of image i,
  // chunk kc, half h of a staged row.  B: lane (j, h) of chunk kc starts at
  // element e = 16 kc + 8 h - j + PW + 32 of its channel's band row.
  const int li = lane & 31, lh = lane >> 5;
  const int a_lane = wave * 4 * HP + lh * HP + li * 16;
  auto read_a = [&](int q, int kc) -> mf_u32x4 {
    return *(const mf_u32x4*)(ring + (q % kBatchSlots) * SLOT + a_lane + 2 * kc * HP);
  };
  const int e0 = 8 * lh - li + a.PW + 32;  // element of chunk 0; chunk 1 is 16 further
  const uint32_t bshift = (uint32_t)(e0 & 1) * 16u;
  const uint32_t* zrow0 = (const uint32_t*)(zt + wave * zrows * ZROW + (e0 & ~1));
  auto read_b = [&](int fh, int kc) -> mf_u32x4 {
    const uint32_t* p = zrow0 + fh * (ZROW / 2) + 8 * kc;
    mf_u32x4 d;
    __builtin_memcpy(&d, p, 16);
    const uint32_t d4 = p[4];
    return mf_u32x4{__builtin_amdgcn_alignbit(d[1], d[0], bshift),
                    __builtin_amdgcn_alignbit(d[2], d[1], bshift),
                    __builtin_amdgcn_alignbit(d[3], d[2], bshift),
                    __builtin_amdgcn_alignbit(d4, d[3], bshift)};
  };

  // Rows of the stream are staged two per barrier, loaded PD barriers
  // ahead: pf[k] holds the two rows of a batch in flight.
  constexpr int PD = kBatchPrefetch;
  Stage pf[PD][2];
#pragma unroll
  for (int k = 0; k < PD; ++k) {
    stage_load(rs, 2 * k, pf[k][0]);
    stage_load(rs, 2 * k + 1, pf[k][1]);
  }
  {
    mb_f32x16 acc[R];
#pragma unroll
    for (int j = 0; j < R; ++j)
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[j][v] = 0.f;
    mf_u32x4 ringA[2][R];  // stream row q of chunk kc in ringA[kc][q % R]

    // Stream rows q = 0 .. nq - 1 (nq = R + FH - 1); row q completes the
    // operands of filter row fh = q - R + 1.  Batch b (rows 2 b, 2 b + 1)
    // goes to LDS at its barrier, while batch b + PD is loaded.  The loop
    // body covers 2 PD R rows, so that ring and prefetch indices are
    // compile-time.
    for (int q0 = 0; q0 < a.nq; q0 += 2 * PD * R) {
#pragma unroll
      for (int bq = 0; bq < PD * R; ++bq) {  // batches of two rows, q = q0 + 2 bq (+1)
        const int qa = q0 + 2 * bq;
        if (qa >= a.nq) break;              // uniform
        const int k = bq % PD;              // q0 is a multiple of 2 PD
        // slots of rows qa, qa + 1 were last read before the previous barrier
        stage_store(qa, pf[k][0]);
        stage_store(qa + 1, pf[k][1]);
        stage_load(rs, qa + 2 * PD, pf[k][0]);
        stage_load(rs, qa + 2 * PD + 1, pf[k][1]);
        __syncthreads();
#pragma unroll
        for (int u = 0; u < 2; ++u) {
          const int q = qa + u;
          const int slot = (2 * bq + u) % R;  // q % R: q0 is a multiple of R
          if (q >= a.nq) break;
          if (row_ok(q)) {
            ringA[0][slot] = read_a(q, 0);
            ringA[1][slot] = read_a(q, 1);
          }
          const int fh = q - (R - 1);
          if (fh < 0) continue;             // still filling the ring
          const mf_u32x4 b0 = read_b(fh, 0), b1 = read_b(fh, 1);
#pragma unroll
          for (int j = 0; j < R; ++j) {
            // output row oh0 + j reads stream row fh + j = q - (R - 1) + j
            const int r = r_base + fh + j;
            if ((unsigned)r >= (unsigned)a.IH || oh0 + j >= a.OH) continue;  // uniform
            const int s = (2 * bq + u + 1 + j) % R;  // (q - R + 1 + j) % R
            acc[j] = mfma_32x32x16<DT>(ringA[0][s], b0, acc[j]);
            acc[j] = mfma_32x32x16<DT>(ringA[1][s], b1, acc[j]);
          }
        }
      }
    }

    // ---- outputs: registers -> LDS [image][column][channel slot] ->
    // channel-contiguous 16-byte stores, two output rows per pair of
    // barriers where the whole LDS holds them (the band is no longer read).  Lane (j, h), register v holds image
    // 8 (v / 4) + 4 h + v % 4 at column j; half h writes channel slot
    // wave ^ h, so that the two halves of a wave fall on different banks
    // (readers swap the pairs back).
    const int oimgs = min(kBatchImg, a.N - n0);
    constexpr int QU = CB / 4;                // channel quads per pixel
    constexpr int KI = kBatchImg * kBatchMaxCols * QU / NT;  // items per thread, at most
    const int nitems = kBatchImg * a.OW * QU;
    const int row_floats = kBatchImg * a.OW * OPITCH;
    float* const ostage = (float*)lds;
    const bool two = a.two_rows;
    // offsets in floats from the group's first output row of channel c0
    // (32-bit: the planner bounds one image group's output)
    float* const obase = a.out + ((size_t)n0 * a.OH + oh0) * a.OW * a.C + c0;
    const uint32_t row_step = (uint32_t)a.OW * (uint32_t)a.C;  // floats per output row
    auto stage_row = [&](int j, float* dst) {
      if (li < a.OW) {
#pragma unroll
        for (int v = 0; v < 16; ++v) {
          const int img = 8 * (v >> 2) + 4 * lh + (v & 3);
          dst[(img * a.OW + li) * OPITCH + (wave ^ lh)] = acc[j][v];
        }
      }
    };
    auto store_row = [&](int j, const float* src) {
#pragma unroll
      for (int k = 0; k < KI; ++k) {
        const int it = tid + k * NT;
        const int qd = it % QU, pc = it / QU;
        const int img = fast_div(pc, a.ow_magic), col = pc - img * a.OW;
        if (it >= nitems || img >= oimgs) continue;
        const mf_f32x4 v = *(const mf_f32x4*)(src + pc * OPITCH + 4 * qd);
        const mf_f32x4 w = (img & 4) ? mf_f32x4{v[1], v[0], v[3], v[2]} : v;
        const uint32_t og = ((uint32_t)img * (uint32_t)a.OH * (uint32_t)a.OW + (uint32_t)col) *
                                (uint32_t)a.C + 4u * (uint32_t)qd;
        // plain stores: L2 merges the channel blocks' 32-byte pieces of each
        // pixel into whole lines (measured: non-temporal stores of the same
        // pattern ran the 31x31 forward at 280 instead of 196 us)
        *(mf_f32x4*)(obase + (og + (uint32_t)j * row_step)) = w;
      }
    };
#pragma unroll
    for (int j = 0; j < R; j += 2) {
      if (oh0 + j >= a.OH) break;           // uniform
      const bool pair = j + 1 < R && oh0 + j + 1 < a.OH;
      __syncthreads();                      // the staging area is free
      stage_row(j, ostage);
      if (two && pair) stage_row(j + 1, ostage + row_floats);
      __syncthreads();
      store_row(j, ostage);
      if (pair) {
        if (two) {
          store_row(j + 1, ostage + row_floats);
        } else {
          __syncthreads();
          stage_row(j + 1, ostage);
          __syncthreads();
          store_row(j + 1, ostage);
        }
      }
    }
  }
}

}  // namespace dwc
