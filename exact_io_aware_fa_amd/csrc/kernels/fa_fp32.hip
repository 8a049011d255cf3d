// Fused attention forward and backward in float32 (vector ALU), for gfx950.
//
// Same method as the bf16 kernels -- the tiled online-softmax forward of
// page 2 ("4. FlashAttention 深度剖析", 4.3.2) with the per-block update of
// page 1 ("注意力为什么受限于显存带宽：用算术强度与分块把 FlashAttention 推导清楚",
// section 六), and the backward by recomputation from L (page 1 section 八,
// page 2 4.3.4) -- with every step in fp32 and no bf16 rounding. This path
// exists for float32 callers and small problems; it uses the vector ALU, not
// the matrix cores.
//
// Forward: a workgroup owns 64 query rows; four consecutive lanes share one
// row, each holding a quarter of q and of the O accumulator (interleaved
// 16-byte chunks). K/V tiles of 32 keys are staged in LDS.
// Backward: a workgroup owns 64 keys (four lanes per key, holding k, v and the
// dK, dV accumulators); it loops over query tiles of 16 rows staged in LDS,
// writes dS to LDS and adds scale * dS K into dQ with float atomics.
#include "fa_device.h"

namespace fa {

namespace {

constexpr int kThreads = 256;

__device__ __forceinline__ float quad_sum(float x) {
  x += __shfl_xor(x, 1);
  x += __shfl_xor(x, 2);
  return x;
}

__device__ __forceinline__ float dot4(f32x4 a, f32x4 b) {
  return fmaf(a[0], b[0], fmaf(a[1], b[1], fmaf(a[2], b[2], a[3] * b[3])));
}

template <int D, bool CAUSAL, bool SPARSE>
__global__ __launch_bounds__(kThreads) void fwd_fp32_kernel(Params p) {
  constexpr int BR = 64;
  constexpr int BC = 32;
  constexpr int C4 = D / 4;     // float4 chunks per row
  constexpr int NV = D / 16;    // chunks per lane (chunk index sub + 4 i)
  __shared__ f32x4 sK[BC][C4];
  __shared__ f32x4 sV[BC][C4];
  __shared__ int sblk[SPARSE ? kMaxBlocks : 1];

  const int tid = threadIdx.x;
  const int row = tid >> 2;
  const int sub = tid & 3;
  const int t_r = (p.n + BR - 1) / BR;
  int b, hq, qb;
  remap_workgroup(blockIdx.x, gridDim.x, t_r, CAUSAL, p.batch, b, hq, qb);
  // Rows of this batch entry; K and V come from the K/V head this query
  // head uses (grouped heads).
  const Span sp = batch_span(p, b);
  const int n = sp.len;
  if (qb * BR >= n) return;  // past the end of a shorter packed sequence
  const size_t qrow0 = span_row0(p, sp, p.heads, hq);
  const size_t base = qrow0 * D;
  const size_t kvbase = span_row0(p, sp, p.heads_kv, hq / p.group) * D;
  const float* __restrict__ Q = static_cast<const float*>(p.q) + base;
  const float* __restrict__ K = static_cast<const float*>(p.k) + kvbase;
  const float* __restrict__ V = static_cast<const float*>(p.v) + kvbase;
  float* __restrict__ O = static_cast<float*>(p.o) + base;
  const int kv_lim = kv_limit(p, b, n);
  const int q0 = qb * BR;
  const int qi = q0 + row;
  const float cs = p.c;
  const float qsgn = p.q_neg ? -1.f : 1.f;

  f32x4 q4[NV], acc[NV];
#pragma unroll
  for (int i = 0; i < NV; ++i) {
    q4[i] = (qi < n) ? *reinterpret_cast<const f32x4*>(Q + (size_t)qi * D + (sub + 4 * i) * 4) * qsgn
                     : f32x4{};
    acc[i] = f32x4{};
  }
  float m2 = kNegInf, l = 0.f;
  // Keys of this row, [lo_i, hi_i), and the key tiles any row of the
  // workgroup needs (the bounds are non-decreasing in the row).
  const Band<CAUSAL> band = make_band<CAUSAL>(p, n, kv_lim);
  const int lo_i = band.lo(qi), hi_i = band.hi(qi);
  const int q_last = min(q0 + BR, n) - 1;
  const int tb = band.lo(q0) / BC;
  const int te = (band.hi(q_last) + BC - 1) / BC;

  auto sweep = [&](const auto& tiles) {
  for (int m = 0; m < tiles.count; ++m) {
    const int k0 = tiles.tile(m) * BC;
    __syncthreads();
    for (int x = tid; x < BC * C4; x += kThreads) {
      const int kr = x / C4, ch = x % C4;
      const int key = k0 + kr;
      f32x4 kv = f32x4{}, vv = f32x4{};
      if (key < kv_lim) {
        kv = *reinterpret_cast<const f32x4*>(K + (size_t)key * D + ch * 4);
        vv = *reinterpret_cast<const f32x4*>(V + (size_t)key * D + ch * 4);
      }
      sK[kr][ch] = kv;
      sV[kr][ch] = vv;
    }
    __syncthreads();

    float sc[BC];
    float mt = kNegInf;
#pragma unroll
    for (int t = 0; t < BC; ++t) {
      float part = 0.f;
#pragma unroll
      for (int i = 0; i < NV; ++i) part += dot4(q4[i], sK[t][sub + 4 * i]);
      part = quad_sum(part);
      const int key = k0 + t;
      const bool hidden = key < lo_i || key >= hi_i;
      sc[t] = hidden ? kNegInf : part;
      mt = fmaxf(mt, sc[t]);
    }
    const float mt2 = (mt == kNegInf) ? kNegInf : mt * cs;
    const float m2n = fmaxf(m2, mt2);
    const float mref = (m2n == kNegInf) ? 0.f : m2n;
    const float alpha = __builtin_amdgcn_exp2f(m2 - mref);
    m2 = m2n;
    float rs = 0.f;
#pragma unroll
    for (int t = 0; t < BC; ++t) {
      sc[t] = __builtin_amdgcn_exp2f(fmaf(sc[t], cs, -mref));
      rs += sc[t];
    }
    l = fmaf(l, alpha, rs);
#pragma unroll
    for (int i = 0; i < NV; ++i) {
      f32x4 a = acc[i] * alpha;
#pragma unroll
      for (int t = 0; t < BC; ++t) a += sc[t] * sV[t][sub + 4 * i];
      acc[i] = a;
    }
  }
  };
  if constexpr (SPARSE) {
    // One block row of the mask covers the workgroup's rows (BR <= kBlock).
    const int nl = stage_blocks(row_blocks(p, q0 / kBlock), sblk, tid, kThreads, p.nb);
    sweep(sparse_tiles<kBlock / BC>(sblk, nl, tb, te));
  } else {
    sweep(dense_tiles(tb, te));
  }

  if (qi < n) {
    const float inv = l > 0.f ? 1.f / l : 0.f;
#pragma unroll
    for (int i = 0; i < NV; ++i)
      *reinterpret_cast<f32x4*>(O + (size_t)qi * D + (sub + 4 * i) * 4) = acc[i] * inv;
    if (sub == 0)
      p.lse[qrow0 + qi] = l > 0.f ? (m2 + log2f(l)) * kLn2 : kNegInf;
  }
}

template <int D, bool CAUSAL, bool SPARSE>
__global__ __launch_bounds__(kThreads) void bwd_fp32_kernel(Params p) {
  constexpr int BK = 64;
  constexpr int BQ = 16;
  constexpr int C4 = D / 4;
  constexpr int NV = D / 16;
  __shared__ f32x4 sQ[BQ][C4];
  __shared__ f32x4 sdO[BQ][C4];
  __shared__ f32x4 sK[BK][C4];
  __shared__ float sL[BQ], sDv[BQ];
  __shared__ float sdS[BQ][BK + 1];
  __shared__ int sblk[SPARSE ? kMaxBlocks : 1];

  const int tid = threadIdx.x;
  const int kr = tid >> 2;
  const int sub = tid & 3;
  const int t_c = (p.n + BK - 1) / BK;
  // The workgroup owns a key tile of K/V head hk of batch entry b and sweeps
  // the queries of every query head in that K/V head's group in turn.
  int b, hk, kt;
  remap_workgroup(blockIdx.x, gridDim.x, t_c, false, p.batch, b, hk, kt);
  const Span sp = batch_span(p, b);
  const int n = sp.len;
  if (kt * BK >= n) return;  // past the end of a shorter packed sequence
  const size_t kvbase = span_row0(p, sp, p.heads_kv, hk) * D;
  const float* __restrict__ K = static_cast<const float*>(p.k) + kvbase;
  const float* __restrict__ V = static_cast<const float*>(p.v) + kvbase;
  float* __restrict__ dK = static_cast<float*>(p.dk) + kvbase;
  float* __restrict__ dV = static_cast<float*>(p.dv) + kvbase;
  const int kv_lim = kv_limit(p, b, n);
  const int k0 = kt * BK;
  const int key = k0 + kr;
  const float cs = p.c;
  const float qsgn = p.q_neg ? -1.f : 1.f;

  f32x4 k4[NV], v4[NV], dk4[NV], dv4[NV];
#pragma unroll
  for (int i = 0; i < NV; ++i) {
    const bool ok = key < kv_lim;
    k4[i] = ok ? *reinterpret_cast<const f32x4*>(K + (size_t)key * D + (sub + 4 * i) * 4) : f32x4{};
    v4[i] = ok ? *reinterpret_cast<const f32x4*>(V + (size_t)key * D + (sub + 4 * i) * 4) : f32x4{};
    dk4[i] = f32x4{};
    dv4[i] = f32x4{};
  }

  if (k0 < kv_lim) {
    for (int x = tid; x < BK * C4; x += kThreads) {
      const int r = x / C4, ch = x % C4;
      sK[r][ch] = (k0 + r < kv_lim) ? *reinterpret_cast<const f32x4*>(K + (size_t)(k0 + r) * D + ch * 4)
                                    : f32x4{};
    }
    // Queries of this key, [qlo_k, qhi_k), and the query tiles any key of the
    // workgroup needs (the bounds are non-decreasing in the key).
    const Band<CAUSAL> band = make_band<CAUSAL>(p, n, kv_lim);
    const int qlo_k = band.qlo(key), qhi_k = band.qhi(key);
    const int k_last = min(k0 + BK, kv_lim) - 1;
    const int tb = band.qlo(k0) / BQ;
    const int te = (band.qhi(k_last) + BQ - 1) / BQ;
    auto sweep = [&](const auto& tiles) {
    for (int gq = 0; gq < p.group; ++gq) {
      // Work entry of query head hk * group + gq (workspace rows).
      const int bh = b * p.heads + hk * p.group + gq;
      const size_t base = span_row0(p, sp, p.heads, hk * p.group + gq) * D;
      const float* __restrict__ Q = static_cast<const float*>(p.q) + base;
      const float* __restrict__ dO = static_cast<const float*>(p.d_o) + base;
      const float* __restrict__ l2v = p.l2vec + (size_t)bh * p.n_pad;
      const float* __restrict__ dvec = p.dvec + (size_t)bh * p.n_pad;
      float* __restrict__ dQ = static_cast<float*>(p.dq) + base;
      // Each query tile starts on a barrier, so the LDS tiles of the previous
      // head are no longer read when this head's first tile is stored.
      for (int m = 0; m < tiles.count; ++m) {
        const int q0 = tiles.tile(m) * BQ;
        __syncthreads();
        for (int x = tid; x < BQ * C4; x += kThreads) {
          const int r = x / C4, ch = x % C4;
          const int q = q0 + r;
          f32x4 a = f32x4{}, g = f32x4{};
          if (q < n) {
            a = *reinterpret_cast<const f32x4*>(Q + (size_t)q * D + ch * 4) * qsgn;
            g = *reinterpret_cast<const f32x4*>(dO + (size_t)q * D + ch * 4);
          }
          sQ[r][ch] = a;
          sdO[r][ch] = g;
        }
        if (tid < BQ) {
          const int q = q0 + tid;
          sL[tid] = (q < n) ? l2v[q] : 0.f;
          sDv[tid] = (q < n) ? dvec[q] : 0.f;
        }
        __syncthreads();

#pragma unroll 4
        for (int t = 0; t < BQ; ++t) {
          const int q = q0 + t;
          float sp = 0.f, dpp = 0.f;
#pragma unroll
          for (int i = 0; i < NV; ++i) {
            sp += dot4(sQ[t][sub + 4 * i], k4[i]);
            dpp += dot4(sdO[t][sub + 4 * i], v4[i]);
          }
          sp = quad_sum(sp);
          dpp = quad_sum(dpp);
          const bool hidden = q < qlo_k || q >= qhi_k;
          const float pr = hidden ? 0.f : __builtin_amdgcn_exp2f(fmaf(sp, cs, -sL[t]));
          const float ds = pr * (dpp - sDv[t]);
#pragma unroll
          for (int i = 0; i < NV; ++i) {
            dv4[i] += pr * sdO[t][sub + 4 * i];
            dk4[i] += ds * sQ[t][sub + 4 * i];
          }
          if (sub == 0) sdS[t][kr] = ds;
        }
        __syncthreads();

        // dQ[q0 + t][col] += scale * sum_r dS[t][r] K[r][col]; 16 lanes per row.
        {
          const int t = tid >> 4;
          const int q = q0 + t;
          const float* kf = reinterpret_cast<const float*>(&sK[0][0]);
          if (q < n) {
            for (int col = tid & 15; col < D; col += 16) {
              float sum = 0.f;
#pragma unroll 8
              for (int r = 0; r < BK; ++r) sum = fmaf(sdS[t][r], kf[r * D + col], sum);
              unsafeAtomicAdd(&dQ[(size_t)q * D + col], p.scale * sum);
            }
          }
        }
      }
    }  // query heads of the group
    };
    if constexpr (SPARSE) {
      // One block column of the mask covers the workgroup's keys (BK <= kBlock).
      const int nl = stage_blocks(col_blocks(p, k0 / kBlock), sblk, tid, kThreads, p.nb);
      sweep(sparse_tiles<kBlock / BQ>(sblk, nl, tb, te));
    } else {
      sweep(dense_tiles(tb, te));
    }
  }

  if (key < n) {
    const float ks = fabsf(p.scale);
#pragma unroll
    for (int i = 0; i < NV; ++i) {
      *reinterpret_cast<f32x4*>(dK + (size_t)key * D + (sub + 4 * i) * 4) = dk4[i] * ks;
      *reinterpret_cast<f32x4*>(dV + (size_t)key * D + (sub + 4 * i) * 4) = dv4[i];
    }
  }
}

template <int D>
hipError_t launch_fwd_d(const Params& p, hipStream_t s) {
  const long long total = (long long)((p.n + 63) / 64) * p.batch * p.heads;
  dim3 grid((unsigned)total), block(kThreads);
  if (p.blk != nullptr) {
    if (p.causal)
      hipLaunchKernelGGL((fwd_fp32_kernel<D, true, true>), grid, block, 0, s, p);
    else
      hipLaunchKernelGGL((fwd_fp32_kernel<D, false, true>), grid, block, 0, s, p);
  } else if (p.causal) {
    hipLaunchKernelGGL((fwd_fp32_kernel<D, true, false>), grid, block, 0, s, p);
  } else {
    hipLaunchKernelGGL((fwd_fp32_kernel<D, false, false>), grid, block, 0, s, p);
  }
  return hipGetLastError();
}

template <int D>
hipError_t launch_bwd_d(const Params& p, hipStream_t s) {
  const long long total = (long long)((p.n + 63) / 64) * p.batch * p.heads_kv;
  dim3 grid((unsigned)total), block(kThreads);
  if (p.blk != nullptr) {
    if (p.causal)
      hipLaunchKernelGGL((bwd_fp32_kernel<D, true, true>), grid, block, 0, s, p);
    else
      hipLaunchKernelGGL((bwd_fp32_kernel<D, false, true>), grid, block, 0, s, p);
  } else if (p.causal) {
    hipLaunchKernelGGL((bwd_fp32_kernel<D, true, false>), grid, block, 0, s, p);
  } else {
    hipLaunchKernelGGL((bwd_fp32_kernel<D, false, false>), grid, block, 0, s, p);
  }
  return hipGetLastError();
}

}  // namespace

hipError_t launch_fwd_fp32(const Params& p, int d, hipStream_t s) {
  switch (d) {
    case 64: return launch_fwd_d<64>(p, s);
    case 128: return launch_fwd_d<128>(p, s);
    case 256: return launch_fwd_d<256>(p, s);
    default: return hipErrorInvalidValue;
  }
}

hipError_t launch_bwd_fp32(const Params& p, int d, hipStream_t s) {
  switch (d) {
    case 64: return launch_bwd_d<64>(p, s);
    case 128: return launch_bwd_d<128>(p, s);
    case 256: return launch_bwd_d<256>(p, s);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace fa
