// dwc_geom.h -- kernel argument blocks and tile constants of libdwc.
// Plain structs shared by the host planner (no HIP needed) and the kernels.
#pragma once

#include <stdint.h>

namespace dwc {

enum { DT_F32 = 0, DT_BF16 = 1, DT_F16 = 2, DT_E4M3 = 3, DT_E5M2 = 4 };

// Channels per wave: one channel per lane, 64 lanes.  In the channel-last
// layout a wave's load of one pixel is 64 consecutive channels, i.e. one
// 256-byte (fp32) or 128-byte (bf16/fp16) contiguous segment.
constexpr int kWaveChannels = 64;
// AUTO: 16-bit and fp8 operands stay on the sweep kernels up to this
// square filter size (stride 1); the packed matrix-core kernels from above
constexpr int kSweepAutoMaxF = 7;
// ... and on the vector kernels for any filter of at most this many rows
// and columns (stride 1)
constexpr int kVecAutoMaxF = 5;
constexpr int kWavesPerBlock = 4;
constexpr int kBlockThreads = 64 * kWavesPerBlock;

// Filter widths with register-window (direct) kernels; a width between two
// of them runs on the next wider one, widths past 31 on the generic kernels.
// X-macro: DWC_DIRECT_FW_LIST(M) expands M(F) per width.
#define DWC_DIRECT_FW_LIST(M) M(3) M(5) M(7) M(9) M(13) M(17) M(21) M(27) M(31)

// The widest listed width below f (0: none): every filter that runs on the
// f-wide body is wider than this, so its first direct_fw_below(f) + 1 taps
// are real ones.
constexpr int direct_fw_below(int f) {
  int b = 0;
#define DWC_BELOW(F) \
  if (F < f) b = F;
  DWC_DIRECT_FW_LIST(DWC_BELOW)
#undef DWC_BELOW
  return b;
}

// Output columns per lane (forward-type kernel) and per strip (filter-gradient
// kernel) that have instantiations.
#define DWC_FWD_TMW_LIST(M) M(7) M(14)
#define DWC_WGRAD_TJ_LIST(M) M(7) M(14)

// Output rows per lane in the forward-type direct kernel, and dY rows per
// register block in the filter-gradient kernel.
constexpr int kFwdRows = 4;
constexpr int kWgradRows = 4;

// Square filters up to this size with stride 1 run the sweep kernels.
constexpr int kSweepMaxF = 9;
#define DWC_SWEEP_F_LIST(M) M(3) M(5) M(7) M(9)

// Filter rows held in registers at once by both direct kernels for a filter
// of width FW: the whole filter up to 9x9, else a chunk of about 64-81
// registers chosen so that common square filters split with little waste
// (13 -> 5+5+3, 17 -> 3 x 6, 21 -> 3 x 7, 27 -> 3 x 9, 31 -> 2 x 16).
constexpr int filter_row_chunk(int fw) {
  return fw <= 9 ? fw : fw == 13 ? 5 : fw <= 27 ? 3 : 2;
}

// Fused prologue of the forward (the batch normalisation and activation
// that precede a DWC, applied to X as it is read): X' = act(X * scale[c] +
// shift[c]), act = clamp to [lo, hi] (identity, relu, relu6), then t *
// sigmoid(t) when silu is set.  Padding stays zero.  scale == nullptr: no
// prologue.
struct Prologue {
  const float* scale;
  const float* shift;
  float lo, hi;
  int silu;
};
// Filters up to this width take the fused prologue (the vector kernels for
// small filters, where the extra arithmetic fits in idle cycles).
constexpr int kPrologueMaxFw = 9;

// Forward-type kernels: the forward map and the stride-1 data gradient (the
// forward map of dY with the filter turned by 180 degrees).
struct FwdArgs {
  const void* in;    // N x IH x IW x C (X, or dY for the data gradient)
  const void* filt;  // FH x FW x C
  float* out;        // N x OH x OW x C
  int N, IH, IW, C;
  int OH, OW;
  int FH, FW, SH, SW;
  int PH, PW;        // zero padding; negative values crop
  int tiles_w, tiles_h, cblocks;
  int num_items;     // waves of work: N * cblocks * tiles_h * tiles_w
  Prologue pro;      // forward only
};

// Strided data gradient by output phase.  For stride S, the dX pixels whose
// row is a (mod S) and column b (mod S) form a stride-1 correlation of dY
// with the sub-filter of taps (f0h + S k, f0w + S l), where f0h = (a + PH)
// mod S and f0w = (b + PW) mod S.  A wave computes one phase of a tile of
// TR x TMW phase pixels; the S*S phases of a tile are consecutive waves.
// The sub-filter is padded to KM x KM taps (zeros past its real size).
#define DWC_PHASE_KM_LIST(M) M(1) M(2) M(3) M(4) M(5) M(6) M(7) M(8) M(10) M(12) M(14) M(16)
constexpr int kPhaseMaxKm = 16;
constexpr int kPhaseTmw = 7;
struct DgradPhaseArgs {
  const void* dy;    // N x OH x OW x C
  const void* filt;  // FH x FW x C
  float* dx;         // N x IH x IW x C
  int N, IH, IW, C, OH, OW;
  int FH, FW, S, PH, PW;
  int tiles_i, tiles_j;  // tiles over ceil(IH / S) x ceil(IW / S) phase pixels
  int cblocks;
  int num_items;     // waves: N * cblocks * tiles_i * tiles_j * S * S
};

// Sweep kernels (stride 1, square F <= 9): waves walk down R consecutive
// output rows of one image.  Forward-type: one wave per (image, row chunk,
// channel block, column strip).  Filter gradient: a workgroup's 4 waves take
// 4 consecutive (image, row chunk) chunks of one (channel block, strip).
struct SweepArgs {
  const void* in;    // forward-type: X (or dY);  filter gradient: X
  const void* in2;   // forward-type: filter;     filter gradient: dY
  float* out;        // forward-type: Y (or dX);  filter gradient: Z x F x F x C partials
  int N, IH, IW, C;  // dims of `in`
  int OH, OW;        // forward-type: output dims; filter gradient: dY dims
  int F, P, PW;      // filter size, row / column padding (forward-type data
                     // gradient: F-1-pad)
  int tiles_w;       // column strips
  int R, cpi;        // output rows per chunk, chunks per image
  int cbg;           // channel blocks: ceil(C / 64)
  int num_items;     // forward-type: waves; filter gradient: workgroups
  int Z;             // filter gradient: partial slices, tiles_w * ceil(N * cpi / 4)
  Prologue pro;      // forward only
  int hybrid;        // filter gradient of fp16 operands: fp16 sub-unit sums
};

// Filter gradient: partial sums over slices of the N*OH axis.  One
// workgroup (4 waves) per (slice, channel block, filter-row chunk); its waves
// split the slice's (row group, column strip) units and add their sums in
// LDS before one partial is written.
struct WgradArgs {
  const void* x;     // N x IH x IW x C
  const void* dy;    // N x OH x OW x C
  float* ws;         // Z x FH x FW x C partial sums
  int N, IH, IW, C, OH, OW;
  int FH, FW, SH, SW, PH, PW;
  int cblocks, fh_tiles, Z;
  int rows;          // N * OH
  int num_items;     // workgroups: Z * cblocks * fh_tiles
};

// Packed-MFMA forward-type kernel (bf16/fp16 operands, stride 1).  Per
// channel, a 16 x 16 block of outputs -- 16 (output row, 16-column group)
// combinations x 16 consecutive columns -- is one v_mfma_f32_16x16x32 per
// filter row and 16-tap fragment: A holds 32 consecutive input columns per
// combination, B the Toeplitz band of one 16-tap slice of the filter row.
// A workgroup owns CB channels x rblk output rows of one image.
// Packed-MFMA workgroups: 8 waves, up to half of a CU's 160 KiB of LDS (two
// workgroups per CU when the registers allow it).
constexpr int kMfmaMaxLds = 81920;
// MI355X (gfx950): compute units and LDS bytes per compute unit.
constexpr int kCus = 256;
constexpr int kLdsPerCu = 163840;
constexpr int kMfmaWaves = 8;
// Packed fp8 forward-type kernel: channels per workgroup (one 16-byte load
// holds 16 fp8 channels of a pixel), bytes per zero-padded filter fragment
// row (16 zeros, 16 taps) and zero rows after the last one.
constexpr int kMfma8Cb = 16;
constexpr int kZ8Row = 32;
constexpr int kZ8Tail = 2;

// Multiplier m = ceil(2^32 / d) with which floor(p / d) = (p * m) >> 32 for
// all p, d < 2^16: writing p = q d + r, p m / 2^32 = q + (r + p e / 2^32) / d
// with e = m d - 2^32 < d, and p e < 2^32 keeps the fraction below 1.  The
// packed-MFMA kernels split filter tap indices by the runtime filter width
// this way (one 64-bit multiply instead of a division sequence).
inline constexpr uint64_t div_magic(uint32_t d) { return ((1ull << 32) + d - 1) / d; }

struct MfmaArgs {
  const void* in;    // N x IH x IW x C (X, or dY for the data gradient)
  const void* filt;  // FH x FW x C
  float* out;        // N x OH x OW x C
  int N, IH, IW, C, OH, OW;
  int FH, FW, PH, PW;  // PH/PW < 0 crop (data gradient with pad > F-1)
  int gt;            // column groups per tile: 1, 2 or 4 (rows per tile 16 / gt)
  int rt_log;        // log2 of the rows per tile, 4 - log2(gt)
  int rblk;          // output rows per workgroup: tiles * 16 / gt
  int rch, cblk;     // row chunks per image, channel blocks
  int xr, wt, wp;    // staged input tile: rows, columns, row pitch (elements)
  int e_items;       // staging lanes per row: (wt / 2) column pairs x CB / 8 octets
  int e2, e2_log;    // e_items rounded up to a power of two, and its log2
  int lds_bytes;
  int num_blocks;    // N * cblk * rch workgroups
  uint64_t fw_magic;  // div_magic(FW): filter tap -> (row, column)
};

// Packed-MFMA forward-type kernel with the batch in the matrix rows (bf16 /
// fp16 operands, stride 1, input and output widths up to 32): per channel,
// output row, filter row and 16-column input chunk, one
// v_mfma_f32_32x32x16 computes 32 images x 32 output columns against the
// Toeplitz band of the filter row.  A workgroup owns kBatchCb channels (one
// per wave) x kBatchImg images x kBatchRows output rows.
constexpr int kBatchCb = 8;
constexpr int kBatchImg = 32;
constexpr int kBatchRows = 7;
// Input rows in flight in LDS (two per barrier), and bytes per staged
// (channel, chunk, 8-column half) plane -- 32 images x 16 bytes and a
// 64-byte pad, so that the four planes a wave's staging writes touch start
// 16 banks apart.
constexpr int kBatchSlots = 4;
// Batches of two input rows loaded ahead of the one being staged.
constexpr int kBatchPrefetch = 1;
constexpr int kBatchHalfPitch = kBatchImg * 16 + 64;
constexpr int kBatchMaxCols = 32;
// AUTO takes the batch-packed kernel from this filter height on; below it
// the row-packed kernel is as fast or faster at N=128 28x28 C=512 (bf16
// 7x7-15x15: 101-120 against 103-127 us for the 16-image kernel; fp16
// 13x13: 114-120 against 121-124 us, 163-167 for the 32-image one), its
// matrix cores being idle either way.
constexpr int kBatchMinFh = 17;
// ... from this height on for outputs at most 16 wide (bf16 N=64 14x14
// C=512 15x15: 22 against 34 us).
constexpr int kBatchMinFhNarrow = 14;
constexpr int kBatchNarrowOw = 16;
// ... and from this height on where its workgroups make a single round of
// at least 3/4 of the CUs (one workgroup per CU: no second workgroup's
// start-up or output phase to wait for; bf16 28x28 with 256 workgroups,
// N=64 C=256 5x5-15x15 and N=32 C=512 9x9-13x13: 26-34 against 31-38 us;
// with 512 or 1024 workgroups, or 128, slower than the row-packed kernel).
constexpr int kBatchMinFhRound = 5;
// ... for fp8 operands, where it takes the 16-image kernel from this filter
// height on (e4m3, N=128 28x28 C=512 5x5-15x15: 85-109 against 103-125 us
// for the row-packed kernel; N=64 28x28 C=256 9x9-15x15: 26-30 against
// 32-34 us).
constexpr int kBatchMinFh8 = 5;
// The same packing with 16 images per v_mfma_f32_16x16x32 and two channels
// per wave: a workgroup owns kB16Cb channels x kB16Img images x kB16Rows
// output rows.  Staged rows: per channel, 4 column groups of 16 images x 16
// bytes; the pitches (kB16KqPitch bytes per column group, kB16ChPitch per
// channel) put the 64 dword writes of one staging instruction on 64
// different banks.  Staged outputs: kB16Opitch floats per pixel (16
// channels and a pad that keeps every pixel 16-byte aligned).
constexpr int kB16Cb = 16;
constexpr int kB16Img = 16;
constexpr int kB16Rows = 7;
constexpr int kB16Slots = 4;
// Batches of two input rows loaded ahead of the one being staged.
constexpr int kB16Prefetch = 1;
constexpr int kB16KqPitch = kB16Img * 16 + 32;
constexpr int kB16ChPitch = 4 * kB16KqPitch + 16;
constexpr int kB16Opitch = 20;
// fp8 operands: 8-byte groups, 16 images x 8 bytes per column group; the
// pitches put the 64 dword writes of one staging instruction (lanes of 4
// images x 16 column pairs x 2 channel halves) on 64 different banks.
constexpr int kB16KqPitch8 = 160;
constexpr int kB16ChPitch8 = 4 * kB16KqPitch8 + 16;
// Filter-tap items (16-byte loads) per thread at the largest filter the
// 16-image kernel takes (FH <= 64, FW <= 32: 2 * 64 * 32 items over 512
// threads).
constexpr int kB16TapItems = 8;
struct MfmaBatchArgs {
  const void* in;    // N x IH x IW x C (X, or dY for the data gradient)
  const void* filt;  // FH x FW x C
  float* out;        // N x OH x OW x C
  int N, IH, IW, C, OH, OW;
  int FH, FW, PH, PW;  // 0 <= PW <= 31, PH >= 0
  int cb;              // channels per workgroup (one per wave): kBatchCb
  int rch, cblk, ng;   // row chunks (OH / kBatchRows), channel blocks, image groups
  int nq;              // input rows streamed per workgroup: kBatchRows + FH - 1
  int two_rows;        // the whole LDS holds two output rows' staging
  int orows;           // output rows staged per round (16-image kernel)
  uint64_t ow_magic;   // div_magic(OW): staged pixel -> (image, column)
  int lds_bytes;
  int num_blocks;      // ng * cblk * rch workgroups
  uint64_t fw_magic;   // div_magic(FW): filter tap -> (row, column)
};

// fp32 matrix-core forward-type kernel (fwd_mfma_f32, stride 1, fp32
// operands): v_mfma_f32_4x4x1_16b_f32 runs 16 independent 4 x 4 outer
// products per instruction.  Block b is channel c0 + b, its 4 rows are 4
// consecutive output rows, its 4 columns 4 consecutive output columns, and
// the K step is one input column: a wave owns 16 channels x 4 output rows
// x 4T output columns of one image.  The filter band (per filter row:
// three zeros, the taps, zeros up to FWI + 3) sits in LDS, shared by the
// workgroup's waves, which all take the same 16 channels.
// Instantiated band widths (FWI); a filter of width FW <= 31 runs on the
// smallest FWI >= FW, the missing taps being zeros.
#define DWC_F32M_FW_LIST(M) M(13) M(17) M(21) M(27) M(31)
#define DWC_F32M_T_LIST(M) M(2) M(4) M(7)
constexpr int kF32mCb = 16;         // channels per wave (the 16 blocks)
constexpr int kF32mRows = 4;        // output rows per wave (the matrix rows)
constexpr int kF32mMaxWaves = 8;    // waves per workgroup
constexpr int kF32mMinFh = 13;      // AUTO: from this many filter rows and columns
constexpr int kF32mMinFPad = 10;    // ... and at any output width for filters from
                                    // this size whose columns stop short of 13
constexpr int kF32mMinOw = 24;      // ... on outputs at least this wide
constexpr int kF32mFillWaves = 2048;  // 8 waves per CU of the MI355X
constexpr int kF32mStageBatch = 8;  // 16-byte band loads in flight per thread
constexpr int f32m_fwi(int fw) {
  return fw <= 13 ? 13 : fw <= 17 ? 17 : fw <= 21 ? 21 : fw <= 27 ? 27 : fw <= 31 ? 31 : 0;
}
// 16-bit forward-type kernel on the 4x4x4 matrix instructions with 4 images
// as the matrix rows (fwd_mfma_h4n; arguments: MfmaF32Args with 16-bit X
// and filter): instantiated band widths and 4-column tiles per wave.
#define DWC_H4M_FW_LIST(M) M(9) M(13) M(17)
#define DWC_H4M_T_LIST(M) M(4) M(7)
constexpr int kH4mCb = 16;         // channels per wave (the 16 blocks)
constexpr int kH4mRows = 4;        // output rows per wave (the accumulator ring)
constexpr int kH4mMaxWaves = 8;    // waves per workgroup
constexpr int kH4mStageBatch = 4;  // band entries (4 two-byte loads each) in flight per thread
constexpr int kH4mMinF = 9;        // AUTO: filters from this many rows and columns
constexpr int kH4mMaxF = 13;       // ... up to this many columns
constexpr int kH4mMaxOw = 16;      // ... on outputs at most this wide
constexpr int kH4mFillWaves = 2048;  // ... with 8 waves per CU of the MI355X
constexpr int h4m_fwi(int fw) { return fw <= 9 ? 9 : fw <= 13 ? 13 : fw <= 17 ? 17 : 0; }
struct MfmaF32Args {
  const void* in;    // N x IH x IW x C fp32 (X, or dY for the data gradient);
                     // bf16/fp16 for fwd_mfma_h4n
  const void* filt;  // FH x FW x C, the same type
  float* out;        // N x OH x OW x C
  int N, IH, IW, C, OH, OW;
  int FH, FW, PH, PW;
  int cblk;          // channel blocks of kF32mCb
  int rg, cg;        // row groups (OH / 4) and column groups (OW / 4T) per image
  int tiles;         // N * rg * cg wave tiles per channel block
  int nw;            // waves per workgroup
  int same;          // PW == (FWI - 1) / 2, FW == FWI and IW == OW: the first and
                     // last column groups skip their padding columns
  int groups;        // workgroups per channel block: ceil(tiles / nw)
  int lds_bytes;     // FH x (FWI + 6) x 16 floats; fwd_mfma_h4n: FH x S x 64 x 8 bytes
  int num_blocks;    // cblk * groups
  uint64_t fw_magic; // div_magic(FW): filter tap -> (row, column)
};

// fp32 matrix-core filter gradient (wgrad_mfma_f32, stride 1): per block
// b (channel c0 + b) of v_mfma_f32_4x4x1_16b_f32,
//   D[i][j] = dW[4h + j][4f + i] += x[r][ow + 4f + i - PW] * dy[r - 4h - j + PH][ow]
// over the K steps (image, input row r, output column ow).  A wave owns one
// filter-row tile h (4 rows) and every column tile f < TW of a channel
// block, over OWW = 4 NB output columns; a workgroup's waves are the
// ceil(FH / 4) row tiles, sharing one staged X row at a time (LDS, double
// buffered); each wave keeps its 4 dY rows per output column in registers,
// moved down a lane quad per input row.  Slices of consecutive (image,
// input row) pairs, times the column groups, write channel-blocked partials
// (cb = 16) that reduce_partials sums.
#define DWC_WF32_TW_LIST(M) M(1) M(2) M(3) M(4) M(5) M(6) M(7) M(8)
#define DWC_WF32_NB_LIST(M) M(2) M(4) M(7) M(14)
constexpr int kWf32Cb = 16;          // channels per workgroup (the 16 blocks)
constexpr int kWf32MaxWaves = 8;     // FH <= 32
constexpr int kWf32StageItems = 2;   // 16-byte X staging items per thread, at most
constexpr int kWf32MinF = 10;        // AUTO: from this filter size (rows and columns)
struct WgradF32Args {
  const void* x;     // N x IH x IW x C fp32, bf16 or fp16
  const void* dy;    // N x OH x OW x C, the same type
  float* ws;         // (Z * cg) x cblk x (FH * FW) x 16 partial sums
  int N, IH, IW, C, OH, OW;
  int FH, FW, PH, PW;
  int cblk, cg, Z;   // channel blocks, column groups, row slices
  int rps;           // (image, input row) pairs per slice
  int nw;            // waves per workgroup: filter-row tiles
  int lds_bytes;
  int num_blocks;    // cblk * cg * Z
};

// out[i] = sum_{z < Z} ws[z * M + j(i)], summed in order of z.  Plain
// layout (cb = 0): j(i) = i.  Channel-blocked layout (cb > 0, C % cb == 0,
// out = [tap][c] with C channels): each slice is [c / cb][tap][c % cb], so
// j(i) = ((c / cb) * taps + tap) * cb + c % cb.
struct ReduceArgs {
  const float* ws;
  float* out;
  int64_t M;
  int Z;
  int cb, C, taps;
};

// Packed-MFMA filter-gradient kernel (bf16/fp16 operands, stride 1).  Per
// channel and output row oh, dW[fh][fw] += sum_i dY[oh][i - fw + pw] *
// X[oh + fh - ph][i]: a v_mfma_f32_16x16x32 with A = the Toeplitz band of
// the dY row (16 taps fw x 32 input columns i) and B = 16 input rows (fh) x
// the same 32 columns.  A workgroup owns kWgmCb channels (one per wave) and
// a slice of images; it writes one partial per slice in the channel-blocked
// layout that reduce_partials reads with cb = kWgmCb.
constexpr int kWgmCb = 8;
// Slices of the packed filter gradients (wgm_slices): partial bytes of all
// slices at most this fraction of the operands' bytes, and about this many
// rounds of resident workgroups
constexpr double kWgmPartFrac = 1.0 / 6.0;
constexpr double kWgmFill = 4.0;
// Staging items (pairs of pixels of one row, kWgmCb channels) per thread
// that a workgroup holds in registers while the previous image computes.
constexpr int kWgmMaxPf = 2;
// Waves per SIMD the filter-gradient kernel is compiled for (its register
// budget: 512 VGPRs / waves): three 8-wave workgroups per CU (80 VGPRs)
// while the fragments and one staging item per thread fit, else two (128),
// else one.
constexpr int wgm_waves_per_eu(int nfm, int nfn, int nk, int pf) {
  return pf == 1 ? ((nk == 1 || nfm * nfn == 1) ? 6 : 4) : (nfm * nfn * nk == 8 ? 2 : 4);
}
// The same for the fp8 kernel: two 8-wave workgroups per CU (128 VGPRs)
// with one staging item per thread, else one.
constexpr int wgm8_waves_per_eu(int pf) { return pf == 1 ? 4 : 2; }
struct WgradMfmaArgs {
  const void* x;     // N x IH x IW x C
  const void* dy;    // N x OH x OW x C
  float* ws;         // Z x cblk x (FH * FW) x kWgmCb partial sums
  int N, IH, IW, C, OH, OW;
  int FH, FW, PH, PW;
  int cblk, Z, ipb;  // channel blocks, slices, images per slice
  int xr, xp;        // staged X: rows (IH + 1, row 0 = zeros), pitch (elements)
  int dyp, dpad;     // staged dY rows: pitch, zeros before column 0
  int hx, ix;        // X items: pixel pairs per row ((IW + 1) / 2), IH * hx
  int e_lo, hd, id;  // dY items: first staged pair, pairs per row, OH * hd
  int lds_bytes;
  int num_blocks;    // Z * cblk
};

// Generic kernels: one output element per lane.
struct GenericArgs {
  const void* a;     // forward / data gradient: X or dY; filter gradient: X
  const void* b;     // forward / data gradient: W;       filter gradient: dY
  float* out;        // Y, dX, or Z x FH x FW x C partial sums
  int N, IH, IW, C, OH, OW;
  int FH, FW, SH, SW, PH, PW;
  int Z, rows;       // filter gradient split
  int64_t total;     // elements (or work items) to produce
};

}  // namespace dwc
