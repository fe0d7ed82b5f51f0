// inst_generic.hip -- generic kernels (any filter size / stride) and the
// deterministic reduction of filter-gradient partials.
#include "dwc_kernels.h"
#include "dwc_launch.h"

#include <type_traits>

namespace dwc {

// Sum of the Z <= kReduceSplitZ slice partials in slice order,
// (((0 + p_0) + p_1) + ...): deterministic for a given split.  A thread owns V consecutive elements of
// the partials' layout (V = 4 where 16-byte accesses line up), with up to
// eight slices' loads in flight; every slice is read in whole contiguous
// rows.  With Z = 0 it writes zeros (the filter gradient of an empty
// batch).  Partials in the channel-blocked layout (cb > 0) go to the
// permuted index of ReduceArgs; with V = 4 the four elements are four
// consecutive channels of one tap.
typedef float rd_f32x4 __attribute__((ext_vector_type(4)));
constexpr int kReduceThreads = 256;

template <int V>
__global__ __launch_bounds__(kReduceThreads) void reduce_partials(ReduceArgs a) {
  typedef typename std::conditional<V == 4, rd_f32x4, float>::type T;
  const int64_t j = ((int64_t)blockIdx.x * kReduceThreads + threadIdx.x) * V;
  if (j >= a.M) return;
  const float* p = a.ws + j;
  T s = T(0.f);
  int z = 0;
  for (; z + 8 <= a.Z; z += 8) {
    T v[8];
#pragma unroll
    for (int k = 0; k < 8; ++k) v[k] = *(const T*)(p + (int64_t)(z + k) * a.M);
#pragma unroll
    for (int k = 0; k < 8; ++k) s += v[k];
  }
  for (; z < a.Z; ++z) s += *(const T*)(p + (int64_t)z * a.M);
  int64_t i = j;
  if (a.cb > 0) {
    const int blk_elems = a.taps * a.cb;  // one channel block's partial: [tap][cb]
    const int cbk = (int)(j / blk_elems), rem = (int)(j - (int64_t)cbk * blk_elems);
    const int tap = rem / a.cb, c = cbk * a.cb + rem - tap * a.cb;
    i = (int64_t)tap * a.C + c;
  }
  *(T*)(a.out + i) = s;
}

// The same sum for many slices (Z > kReduceSplitZ) over few elements: a
// block of 16 waves owns 64 consecutive elements (one per lane); wave w
// adds the contiguous slice range [w Z / 16, (w + 1) Z / 16) in slice
// order, then wave 0 adds the 16 wave sums in wave order (deterministic as
// well, with the association that split fixes).
constexpr int kReduceWaves = 16;
constexpr int kReduceSplitZ = 32;

__global__ __launch_bounds__(64 * kReduceWaves) void reduce_partials_split(ReduceArgs a) {
  __shared__ float part[kReduceWaves][64];
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int64_t j = (int64_t)blockIdx.x * 64 + lane;
  int64_t i = j;
  if (a.cb > 0 && j < a.M) {
    const int blk_elems = a.taps * a.cb;  // one channel block's partial: [tap][cb]
    const int cbk = (int)(j / blk_elems), rem = (int)(j - (int64_t)cbk * blk_elems);
    const int tap = rem / a.cb, c = cbk * a.cb + rem - tap * a.cb;
    i = (int64_t)tap * a.C + c;
  }
  const int z0 = (int)((int64_t)a.Z * wave / kReduceWaves);
  const int z1 = (int)((int64_t)a.Z * (wave + 1) / kReduceWaves);
  float s = 0.f;
  if (j < a.M) {
    const float* p = a.ws + j;
    int z = z0;
    for (; z + 8 <= z1; z += 8) {
      float v[8];
#pragma unroll
      for (int k = 0; k < 8; ++k) v[k] = p[(int64_t)(z + k) * a.M];
#pragma unroll
      for (int k = 0; k < 8; ++k) s += v[k];
    }
    for (; z < z1; ++z) s += p[(int64_t)z * a.M];
  }
  part[wave][lane] = s;
  __syncthreads();
  if (wave == 0 && j < a.M) {
    float t = 0.f;
#pragma unroll
    for (int w = 0; w < kReduceWaves; ++w) t += part[w][lane];
    a.out[i] = t;
  }
}

namespace {

template <int DT>
hipError_t generic_dt(int kind, const GenericArgs& a, hipStream_t s) {
  const int64_t blocks = (a.total + 255) / 256;
  if (blocks == 0) return hipSuccess;
  if (blocks > 0x7fffffff) return hipErrorInvalidValue;
  switch (kind) {
    case GEN_FWD:
      hipLaunchKernelGGL((fwd_generic<DT, false>), dim3((unsigned)blocks), dim3(256), 0, s, a);
      break;
    case GEN_FWD_FLIP:
      hipLaunchKernelGGL((fwd_generic<DT, true>), dim3((unsigned)blocks), dim3(256), 0, s, a);
      break;
    case GEN_DGRAD:
      hipLaunchKernelGGL((dgrad_generic<DT>), dim3((unsigned)blocks), dim3(256), 0, s, a);
      break;
    case GEN_WGRAD:
      hipLaunchKernelGGL((wgrad_generic<DT>), dim3((unsigned)blocks), dim3(256), 0, s, a);
      break;
    default:
      return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace

hipError_t launch_generic(int kind, int dt, const GenericArgs& a, hipStream_t s) {
  switch (dt) {
    case DT_F32: return generic_dt<DT_F32>(kind, a, s);
    case DT_BF16: return generic_dt<DT_BF16>(kind, a, s);
    case DT_F16: return generic_dt<DT_F16>(kind, a, s);
    case DT_E4M3: return generic_dt<DT_E4M3>(kind, a, s);
    case DT_E5M2: return generic_dt<DT_E5M2>(kind, a, s);
  }
  return hipErrorInvalidValue;
}

hipError_t launch_reduce(const ReduceArgs& a, hipStream_t s) {
  if (a.Z > kReduceSplitZ) {
    const int64_t blocks = (a.M + 63) / 64;
    if (blocks == 0) return hipSuccess;
    hipLaunchKernelGGL(reduce_partials_split, dim3((unsigned)blocks), dim3(64 * kReduceWaves), 0,
                       s, a);
    return hipGetLastError();
  }
  // four elements per thread where every 16-byte access is aligned and, in
  // the channel-blocked layout, four consecutive elements are four
  // consecutive channels of one tap
  const bool v4 = a.M % 4 == 0 && (uintptr_t)a.ws % 16 == 0 && (uintptr_t)a.out % 16 == 0 &&
                  (a.cb == 0 || (a.cb % 4 == 0 && a.C % 4 == 0));
  const int64_t threads = v4 ? a.M / 4 : a.M;
  const int64_t blocks = (threads + kReduceThreads - 1) / kReduceThreads;
  if (blocks == 0) return hipSuccess;
  if (v4)
    hipLaunchKernelGGL(reduce_partials<4>, dim3((unsigned)blocks), dim3(kReduceThreads), 0, s, a);
  else
    hipLaunchKernelGGL(reduce_partials<1>, dim3((unsigned)blocks), dim3(kReduceThreads), 0, s, a);
  return hipGetLastError();
}

}  // namespace dwc
