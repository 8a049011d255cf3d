// Attention backward, dK/dV part, register-staged variant (used for d = 256).
//
// Same method and wave layout as fa_bwd_bf16.hip (page 1, "注意力为什么受限于
// 显存带宽：用算术强度与分块把 FlashAttention 推导清楚", section 八; page 2,
// "4. FlashAttention 深度剖析", 4.3.4): a workgroup owns 128 keys (32 per
// wave) and their dK, dV accumulators for the whole query sweep; K and V rows
// are B operands held in VGPRs; P and dS stay in registers as B operands of
// dV^T += dO^T P and dK^T += Q^T dS. The difference is how the query tiles
// reach LDS: each thread loads 16-byte chunks into registers and writes
// every tile twice, row-major (rows padded by 16 bytes) and transposed
// ([d][query], rows padded by 8 bytes, built with byte permutes), one tile
// at a time. At d = 256 the dK and dV accumulators alone take 256 registers,
// which leaves no room for the software pipeline of the d <= 128 kernel.
// S and dP accumulate in VGPRs (mma32_v, mma32_v0 in fa_device.h; the
// compiler would give the AGPR form to every product of a kernel this size,
// and the vector units would then move each value out of and back into
// AGPRs); mfma_drain waits for the last of them before S and dP are read.
#include <type_traits>

#include "fa_device.h"

namespace fa {

namespace {

constexpr int kThreads = 256;
constexpr int kBKV = 128;  // keys per workgroup (4 waves x 32)

template <int D, int BQ, int NBUF, bool CAUSAL, bool SPARSE>
__global__ __launch_bounds__(kThreads, 1) void bwd_dkdv_staged_kernel(Params p) {
  constexpr int ND = D / 16;
  constexpr int NMB = D / 32;
  constexpr int NQB = BQ / 32;
  constexpr int QSTR = D + 8;      // row-major Q / dO tiles
  constexpr int TSTR = BQ + 4;     // transposed tiles [d][q]
  constexpr int UPT = (BQ / 4) * (D / 8);  // 4x8 units per tensor tile
  constexpr int UNITS = 2 * UPT;           // Q and dO
  constexpr int UPTH = (UNITS + kThreads - 1) / kThreads;
  static_assert(UNITS % kThreads == 0, "unit split");

  // NBUF = 2: the Q/dO tiles, their transposes and L/D are double
  // buffered, so one barrier per query tile suffices (see the loop below).
  __shared__ __attribute__((aligned(16))) bf16 sQ[NBUF][BQ * QSTR];
  __shared__ __attribute__((aligned(16))) bf16 sdO[NBUF][BQ * QSTR];
  __shared__ __attribute__((aligned(16))) bf16 sQt[NBUF][D * TSTR];
  __shared__ __attribute__((aligned(16))) bf16 sdOt[NBUF][D * TSTR];
  __shared__ __attribute__((aligned(16))) float sL[NBUF][BQ];
  __shared__ __attribute__((aligned(16))) float sDv[NBUF][BQ];
  __shared__ int sblk[SPARSE ? kMaxBlocks : 1];

  const int tid = threadIdx.x;
  const int w = tid >> 6;
  const int lane = tid & 63;
  const int c = lane & 31;
  const int h = lane >> 5;

  const int t_c = (p.n + kBKV - 1) / kBKV;
  // The workgroup owns a key tile of K/V head hk of batch entry b and sweeps
  // the queries of every query head in that K/V head's group in turn.
  int b, hk, kt;
  remap_workgroup(blockIdx.x, gridDim.x, t_c, false, p.batch, b, hk, kt);
  const Span sp = batch_span(p, b);
  const int n = sp.len;
  if (kt * kBKV >= n) return;  // past the end of a shorter packed sequence
  const size_t kvbase = span_row0(p, sp, p.heads_kv, hk) * D;
  const bf16* __restrict__ K = static_cast<const bf16*>(p.k) + kvbase;
  const bf16* __restrict__ V = static_cast<const bf16*>(p.v) + kvbase;
  bf16* __restrict__ dK = static_cast<bf16*>(p.dk) + kvbase;
  bf16* __restrict__ dV = static_cast<bf16*>(p.dv) + kvbase;
  // Q, dO and the row vectors of the query head being swept.
  const bf16* __restrict__ Q = nullptr;
  const bf16* __restrict__ dO = nullptr;
  const float* __restrict__ l2v = nullptr;
  const float* __restrict__ dvec = nullptr;

  const int kv_lim = kv_limit(p, b, n);
  const int k0 = kt * kBKV;
  const int kw0 = k0 + w * 32;
  const int mykey = kw0 + c;
  const float cs = p.c;
  // A negative scale is applied by negating K (exact in bf16): the scores
  // use K' = -K with |scale|, and dK = scale dS^T Q with the true Q.
  const uint32_t kflip = p.q_neg ? 0x80008000u : 0u;

  f32x16 dk[NMB], dv[NMB];
#pragma unroll
  for (int mb = 0; mb < NMB; ++mb) {
    dk[mb] = f32x16{};
    dv[mb] = f32x16{};
  }

  if (k0 < kv_lim) {
    // K and V rows of this wave as B fragments: [mykey][kd*16 + h*8 + e].
    // Rows past the key limit are read clamped and replaced by zeros.
    bf16x8 kf[ND], vf[ND];
    {
      const bool kok = mykey < kv_lim;
      const int kr = kok ? mykey : kv_lim - 1;
#pragma unroll
      for (int kd = 0; kd < ND; ++kd) {
        const u32x4 z = {0u, 0u, 0u, 0u};
        const u32x4 a = ld16(K + (size_t)kr * D + kd * 16 + h * 8);
        const u32x4 bb = ld16(V + (size_t)kr * D + kd * 16 + h * 8);
        kf[kd] = as_bf16x8(kok ? (a ^ kflip) : z);
        vf[kd] = as_bf16x8(kok ? bb : z);
      }
    }
    // Queries that see this lane's key: [qlo, qhi) (qlo = n for keys at or
    // past the key limit). Query tiles [tb, te) hold every query some key of
    // the workgroup is seen by, tiles [iu0, iu1) only queries that see all
    // of its keys (the bounds are non-decreasing in the key); rows past n
    // are always masked.
    const Band<CAUSAL> band = make_band<CAUSAL>(p, n, kv_lim);
    const int qlo = band.qlo(mykey), qhi = band.qhi(mykey);
    const int k_last = min(k0 + kBKV, kv_lim) - 1;
    const int tb = band.qlo(k0) / BQ;
    const int te = (band.qhi(k_last) + BQ - 1) / BQ;
    const int iu0 = (band.qlo(k0 + kBKV - 1) + BQ - 1) / BQ;
    const int iu1 = band.qhi(k0) / BQ;

    // Register staging of the next Q / dO tile: unit u < UPT is a Q unit,
    // else a dO unit; a unit is 4 rows x 8 dims. Rows past n are read
    // clamped to row n-1; every product involving them is masked (P = 0,
    // dS = 0) and their dQ rows are not written.
    // L and D of the tile's queries travel with it (loaded here, one tile
    // ahead, rather than when the tile is written to LDS, where the write
    // would wait for them).
    u32x4 ureg[UPTH][4];
    float lreg = 0.f, dreg = 0.f;
    auto gload = [&](int it) {
      const int q0 = it * BQ;
      if (tid < BQ) {
        const int q = min(q0 + tid, n - 1);
        lreg = l2v[q];
        dreg = dvec[q];
      }
#pragma unroll
      for (int i = 0; i < UPTH; ++i) {
        const int u0 = tid + i * kThreads;
        const bool isq = u0 < UPT;
        const int u = isq ? u0 : u0 - UPT;
        const int qg = (u >> 2) % (BQ / 4);
        const int dg = (u & 3) + 4 * (u / BQ);
        const bf16* src = (isq ? Q : dO) + dg * 8;
#pragma unroll
        for (int t = 0; t < 4; ++t)
          ureg[i][t] = ld16(src + (size_t)min(q0 + qg * 4 + t, n - 1) * D);
      }
    };
    auto swrite = [&](int it, int buf) {
#pragma unroll
      for (int i = 0; i < UPTH; ++i) {
        const int u0 = tid + i * kThreads;
        const bool isq = u0 < UPT;
        const int u = isq ? u0 : u0 - UPT;
        const int qg = (u >> 2) % (BQ / 4);
        const int dg = (u & 3) + 4 * (u / BQ);
        bf16* rm = isq ? sQ[buf] : sdO[buf];
        bf16* tr = isq ? sQt[buf] : sdOt[buf];
#pragma unroll
        for (int t = 0; t < 4; ++t)
          *reinterpret_cast<u32x4*>(&rm[(qg * 4 + t) * QSTR + dg * 8]) = ureg[i][t];
#pragma unroll
        for (int e = 0; e < 8; ++e)
          *reinterpret_cast<u32x2*>(&tr[(dg * 8 + e) * TSTR + qg * 4]) = column4(ureg[i], e);
      }
      if (tid < BQ) {
        sL[buf][tid] = lreg;
        sDv[buf][tid] = dreg;
      }
    };

    // Tile compute on LDS buffer `buf`: S = Q K^T and dP = dO V^T (lane =
    // key, 16 queries per 32-query block), P = exp2(S c - L log2 e),
    // dS = P (dP - D), then dV^T += dO^T P and dK^T += Q^T dS.
    auto compute = [&](int it, int buf, auto mask_tag) {
      constexpr bool MASK = decltype(mask_tag)::value;
      const int q0 = it * BQ;
      const bf16* tQ = sQ[buf];
      const bf16* tdO = sdO[buf];
      const bf16* tQt = sQt[buf];
      const bf16* tdOt = sdOt[buf];

      // A fragments are read two products ahead through a ring of three (the
      // sched_barrier fences keep the compiler from hoisting every read to
      // the top, which would hold all 2 ND fragments in registers at once).
      f32x16 sv[NQB], dp[NQB];
#pragma unroll
      for (int qb = 0; qb < NQB; ++qb) {
        auto rd = [&](const bf16* t, int kd) FA_INLINE {
          return as_bf16x8(ld16(&t[(qb * 32 + c) * QSTR + kd * 16 + h * 8]));
        };
        bf16x8 qa[3], ga[3];
        qa[0] = rd(tQ, 0);
        ga[0] = rd(tdO, 0);
        qa[1] = rd(tQ, 1);
        ga[1] = rd(tdO, 1);
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int kd = 0; kd < ND; ++kd) {
          if (kd + 2 < ND) {
            qa[(kd + 2) % 3] = rd(tQ, kd + 2);
            ga[(kd + 2) % 3] = rd(tdO, kd + 2);
          }
          if (kd == 0) {
            sv[qb] = mma32_v0(qa[0], kf[0]);
            dp[qb] = mma32_v0(ga[0], vf[0]);
          } else {
            sv[qb] = mma32_v(qa[kd % 3], kf[kd], sv[qb]);
            dp[qb] = mma32_v(ga[kd % 3], vf[kd], dp[qb]);
          }
          __builtin_amdgcn_sched_barrier(0);
        }
      }
      // S and dP are read right below: let the last products finish.
      mfma_drain();
#pragma unroll
      for (int qb = 0; qb < NQB; ++qb)
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          const f32x4 l4 = *reinterpret_cast<const f32x4*>(&sL[buf][qb * 32 + g * 8 + h * 4]);
          const f32x4 d4 = *reinterpret_cast<const f32x4*>(&sDv[buf][qb * 32 + g * 8 + h * 4]);
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const int r = g * 4 + i;
            float pr = __builtin_amdgcn_exp2f(fmaf(sv[qb][r], cs, -l4[i]));
            if (MASK) {
              const int q = q0 + qb * 32 + g * 8 + h * 4 + i;
              const bool hidden = q < qlo || q >= qhi;
              pr = hidden ? 0.f : pr;
            }
            sv[qb][r] = pr;
            dp[qb][r] = pr * (dp[qb][r] - d4[i]);
          }
        }
#pragma unroll
      for (int qb = 0; qb < NQB; ++qb)
#pragma unroll
        for (int qc = 0; qc < 2; ++qc) {
          u32x4 pu, su;
#pragma unroll
          for (int t = 0; t < 4; ++t) {
            pu[t] = pack_bf16x2(sv[qb][qc * 8 + 2 * t], sv[qb][qc * 8 + 2 * t + 1]);
            su[t] = pack_bf16x2(dp[qb][qc * 8 + 2 * t], dp[qb][qc * 8 + 2 * t + 1]);
          }
          const bf16x8 pfr = as_bf16x8(pu);
          const bf16x8 sfr = as_bf16x8(su);
          // Transposed A fragments one pair ahead, as above.
          auto rdt = [&](int mb, bf16x8& fo, bf16x8& fq) FA_INLINE {
            const int off = (mb * 32 + c) * TSTR + qb * 32 + qc * 16 + h * 4;
            const u32x2 olo = ld8(&tdOt[off]);
            const u32x2 ohi = ld8(&tdOt[off + 8]);
            fo = as_bf16x8(u32x4{olo[0], olo[1], ohi[0], ohi[1]});
            const u32x2 qlo = ld8(&tQt[off]);
            const u32x2 qhi = ld8(&tQt[off + 8]);
            fq = as_bf16x8(u32x4{qlo[0], qlo[1], qhi[0], qhi[1]});
          };
          bf16x8 oa[2], qa[2];
          rdt(0, oa[0], qa[0]);
          __builtin_amdgcn_sched_barrier(0);
#pragma unroll
          for (int mb = 0; mb < NMB; ++mb) {
            if (mb + 1 < NMB) rdt(mb + 1, oa[(mb + 1) % 2], qa[(mb + 1) % 2]);
            dv[mb] = mma32(oa[mb % 2], pfr, dv[mb]);
            dk[mb] = mma32(qa[mb % 2], sfr, dk[mb]);
            __builtin_amdgcn_sched_barrier(0);
          }
        }
    };

    auto sweep = [&](const auto& tiles) FA_INLINE {
    const int ns = tiles.count;
    // Steps [su0, su1) hold only queries that see every key of the workgroup.
    const int su0 = tiles.first_at_least(iu0);
    const int su1 = max(tiles.first_at_least(iu1), su0);
    auto run = [&](int it, int buf, auto mask_tag) FA_INLINE {
      // it counts steps; tiles.tile(it) is the query tile of step it.
      const int t = tiles.tile(it);
      if constexpr (NBUF == 2) {
        // Buffer `buf` holds tile t. The next tile goes to buf^1 while t is
        // processed: buf^1 was last read before the previous barrier.
        compute(t, buf, mask_tag);
        if (it + 1 < ns) {
          swrite(tiles.tile(it + 1), buf ^ 1);
          gload(tiles.tile(min(it + 2, ns - 1)));
        }
        __syncthreads();  // next tile complete; buf free for the one after
      } else {
        __syncthreads();  // previous tile's LDS contents are no longer read
        swrite(t, 0);
        __syncthreads();
        gload(tiles.tile(min(it + 1, ns - 1)));
        compute(t, 0, mask_tag);
      }
    };

    // One sweep per query head of the group. A sweep's first LDS write is
    // safe: with two buffers every step ends on a barrier, with one every
    // step starts on one.
    if (ns > 0)
    for (int gq = 0; gq < p.group; ++gq) {
      // Work entry of query head hk * group + gq (workspace rows).
      const int bh = b * p.heads + hk * p.group + gq;
      const size_t base = span_row0(p, sp, p.heads, hk * p.group + gq) * D;
      Q = static_cast<const bf16*>(p.q) + base;
      dO = static_cast<const bf16*>(p.d_o) + base;
      l2v = p.l2vec + (size_t)bh * p.n_pad;
      dvec = p.dvec + (size_t)bh * p.n_pad;
      gload(tiles.tile(0));
      if constexpr (NBUF == 2) {
        swrite(tiles.tile(0), 0);
        gload(tiles.tile(min(1, ns - 1)));
        __syncthreads();
      }
      // Masked steps, unmasked steps (only fully visible queries), masked
      // steps again.
      int it = 0;
      for (; it < su0; ++it) run(it, it & (NBUF - 1), std::true_type{});
      for (; it < su1; ++it) run(it, it & (NBUF - 1), std::false_type{});
      for (; it < ns; ++it) run(it, it & (NBUF - 1), std::true_type{});
    }
    };
    if constexpr (SPARSE) {
      // The workgroup's keys lie in one block column of the mask.
      const int nl = stage_blocks(col_blocks(p, k0 / kBlock), sblk, tid, kThreads, p.nb);
      sweep(sparse_tiles<kBlock / BQ>(sblk, nl, tb, te));
    } else {
      sweep(dense_tiles(tb, te));
    }
  }

  // dK = scale * (dS^T Q), dV as accumulated.
  if (mykey < n) {
    const float ks = p.scale;
#pragma unroll
    for (int mb = 0; mb < NMB; ++mb)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const size_t off = (size_t)mykey * D + mb * 32 + g * 8 + h * 4;
        u32x2 uk, uv;
        uk[0] = pack_bf16x2(dk[mb][g * 4 + 0] * ks, dk[mb][g * 4 + 1] * ks);
        uk[1] = pack_bf16x2(dk[mb][g * 4 + 2] * ks, dk[mb][g * 4 + 3] * ks);
        uv[0] = pack_bf16x2(dv[mb][g * 4 + 0], dv[mb][g * 4 + 1]);
        uv[1] = pack_bf16x2(dv[mb][g * 4 + 2], dv[mb][g * 4 + 3]);
        *reinterpret_cast<u32x2*>(dK + off) = uk;
        *reinterpret_cast<u32x2*>(dV + off) = uv;
      }
  }
}

template <int D, int BQ, int NBUF>
hipError_t launch_d(const Params& p, hipStream_t s) {
  const int t_c = (p.n + kBKV - 1) / kBKV;
  const long long total = (long long)t_c * p.batch * p.heads_kv;
  dim3 grid((unsigned)total), block(kThreads);
  return dispatch_mask(p, [&](auto causal, auto sparse) {
    hipLaunchKernelGGL((bwd_dkdv_staged_kernel<D, BQ, NBUF, decltype(causal)::value,
                                               decltype(sparse)::value>),
                       grid, block, 0, s, p);
    return hipGetLastError();
  });
}

}  // namespace

hipError_t launch_bwd_dkdv_bf16_staged(const Params& p, int d, hipStream_t s) {
  switch (d) {
    case 256: return launch_d<256, 32, 1>(p, s);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace fa
