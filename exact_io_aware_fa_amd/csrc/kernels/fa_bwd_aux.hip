// Backward helper kernels (HBM-bound, no matrix work).
//
// bwd_prep: for every query row, D_i = sum_k dO_ik O_ik in fp32 -- the row
// term of dS = P * (dP - D) (ordinary softmax calculus: sum_j P_ij dP_ij =
// <dO_i, O_i>; the pages name the backward's dS but print no formula) -- and
// L_i log2(e), the saved row statistic in the base-2 units the kernels use.
// Both vectors are written per (batch entry, head) padded to n_pad rows
// (padding and rows past a shorter packed sequence = 0) so the backward
// kernels can load any 64-row slice directly. When an
// accumulator is given (fp32 path) the dQ rows are zeroed as well. D/8 lanes
// share a row, each reading 8 elements (16 bytes for bf16) of O and dO.
#include "fa_device.h"

namespace fa {

namespace {

constexpr int kThreads = 256;

__device__ __forceinline__ void load8(const bf16* p, float out[8]) {
  const u32x4 v = ld16(p);
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    out[2 * i] = __uint_as_float(v[i] << 16);
    out[2 * i + 1] = __uint_as_float(v[i] & 0xffff0000u);
  }
}

__device__ __forceinline__ void load8(const float* p, float out[8]) {
  const f32x4 a = *reinterpret_cast<const f32x4*>(p);
  const f32x4 b = *reinterpret_cast<const f32x4*>(p + 4);
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    out[i] = a[i];
    out[4 + i] = b[i];
  }
}

template <int D, typename T>
__global__ __launch_bounds__(kThreads) void bwd_prep_kernel(Params p, long long rows) {
  constexpr int G = D / 8;            // lanes per row
  constexpr int RPB = kThreads / G;   // rows per block
  const long long row = (long long)blockIdx.x * RPB + threadIdx.x / G;  // padded row
  const int sub = threadIdx.x % G;
  if (row >= rows) return;  // whole G-lane groups leave together
  // Work entry bh = (batch entry, query head) and its row i.
  const int bh = (int)(row / p.n_pad);
  const int i = (int)(row - (long long)bh * p.n_pad);
  const int b = bh / p.heads;
  const Span sp = batch_span(p, b);
  if (i >= sp.len) {
    if (sub == 0) {
      p.dvec[row] = 0.f;
      p.l2vec[row] = 0.f;
    }
    return;
  }
  const size_t qrow = span_row0(p, sp, p.heads, bh - b * p.heads) + i;
  const size_t off = qrow * D + sub * 8;
  float o[8], g[8];
  load8(static_cast<const T*>(p.o_in) + off, o);
  load8(static_cast<const T*>(p.d_o) + off, g);
  float s = 0.f;
#pragma unroll
  for (int k = 0; k < 8; ++k) s = fmaf(o[k], g[k], s);
#pragma unroll
  for (int m = 1; m < G; m <<= 1) s += __shfl_xor(s, m);
  if (sub == 0) {
    p.dvec[row] = s;
    // A row with no visible key (LSE = -inf) gets +inf, so every rebuilt
    // probability exp2(s c - L log2 e) of it is exactly 0.
    const float lse = p.lse[qrow];
    p.l2vec[row] = lse == kNegInf ? __builtin_inff() : lse * kLog2e;
  }
  if (p.dq_acc != nullptr) {
    *reinterpret_cast<f32x4*>(p.dq_acc + off) = f32x4{};
    *reinterpret_cast<f32x4*>(p.dq_acc + off + 4) = f32x4{};
  }
}

template <int D>
hipError_t launch_prep_d(const Params& p, bool is_bf16, hipStream_t s) {
  const long long rows = (long long)p.batch * p.heads * p.n_pad;
  constexpr int RPB = kThreads / (D / 8);
  dim3 grid((unsigned)((rows + RPB - 1) / RPB)), block(kThreads);
  if (is_bf16)
    hipLaunchKernelGGL((bwd_prep_kernel<D, bf16>), grid, block, 0, s, p, rows);
  else
    hipLaunchKernelGGL((bwd_prep_kernel<D, float>), grid, block, 0, s, p, rows);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_bwd_prep(const Params& p, int d, bool is_bf16, hipStream_t s) {
  switch (d) {
    case 64: return launch_prep_d<64>(p, is_bf16, s);
    case 128: return launch_prep_d<128>(p, is_bf16, s);
    case 256: return launch_prep_d<256>(p, is_bf16, s);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace fa
