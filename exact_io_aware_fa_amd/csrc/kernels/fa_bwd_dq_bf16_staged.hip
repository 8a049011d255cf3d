// Attention backward, dQ part, register-staged variant (used for d = 256).
//
// Same method and wave layout as fa_bwd_dq_bf16.hip (page 1, "注意力为什么受限
// 于显存带宽：用算术强度与分块把 FlashAttention 推导清楚", section 八; page 2,
// "4. FlashAttention 深度剖析", 4.3.4): a workgroup owns 128 query rows (32 per
// wave), recomputes S^T and dP^T with Q and dO rows held as B operands, and
// accumulates dQ^T += K^T dS^T in registers. The difference is how key tiles
// reach LDS: each thread loads 16-byte chunks into registers and writes K
// row-major and transposed (byte permutes) and V row-major, one tile at a
// time with two barriers. At d = 256 the dQ accumulator and the Q and dO
// fragments alone fill the register budget of two waves per SIMD.
#include <type_traits>

#include "fa_device.h"

namespace fa {

namespace {

constexpr int kThreads = 256;
constexpr int kBR = 128;  // query rows per workgroup (4 waves x 32)

template <int D, int BC, bool CAUSAL, bool SPARSE, bool WIN>
// One workgroup per CU (one wave per SIMD): the dQ accumulator and the Q
// and dO fragments then fit the 512 registers of a lone wave (with AGPRs);
// at two per CU they spilled 150-700 registers per lane, which cost more
// than the halved occupancy (d = 256 backward 340 -> 490 TFLOP/s).
__global__ __launch_bounds__(kThreads, 1) void bwd_dq_staged_kernel(Params p) {
  constexpr int KSTR = D + 8;    // row-major K / V tiles (bf16 elements)
  constexpr int TSTR = BC + 4;   // transposed K tile [d][key]
  constexpr int ND = D / 16;
  constexpr int NMB = D / 32;
  constexpr int NKB = BC / 32;
  constexpr int KUN = (BC / 4) * (D / 8);  // K units: 4 keys x 8 dims
  constexpr int KUPT = (KUN + kThreads - 1) / kThreads;
  constexpr int VCH = BC * D / 8 / kThreads;  // 16-byte V chunks per thread
  static_assert(VCH * kThreads * 8 == BC * D, "V tile split");
  static_assert(KUN % kThreads == 0 || KUN < kThreads, "K unit split");

  __shared__ __attribute__((aligned(16))) bf16 sK[BC * KSTR];
  __shared__ __attribute__((aligned(16))) bf16 sV[BC * KSTR];
  __shared__ __attribute__((aligned(16))) bf16 sKt[D * TSTR];
  __shared__ int sblk[SPARSE ? kMaxBlocks : 1];

  const int tid = threadIdx.x;
  const int w = tid >> 6;
  const int lane = tid & 63;
  const int c = lane & 31;
  const int h = lane >> 5;

  const int t_r = (p.n + kBR - 1) / kBR;
  int b, hq, qb;
  remap_workgroup(blockIdx.x, gridDim.x, t_r, CAUSAL, p.batch, b, hq, qb);
  const int bh = b * p.heads + hq;  // work entry (workspace rows)
  // Rows of this batch entry; K and V come from the K/V head this query
  // head uses (grouped heads).
  const Span sp = batch_span(p, b);
  const int n = sp.len;
  if (qb * kBR >= n) return;  // past the end of a shorter packed sequence
  const size_t qrow0 = span_row0(p, sp, p.heads, hq);
  const size_t base = qrow0 * D;
  const size_t kvbase = span_row0(p, sp, p.heads_kv, hq / p.group) * D;
  const bf16* __restrict__ Q = static_cast<const bf16*>(p.q) + base;
  const bf16* __restrict__ K = static_cast<const bf16*>(p.k) + kvbase;
  const bf16* __restrict__ V = static_cast<const bf16*>(p.v) + kvbase;
  const bf16* __restrict__ dO = static_cast<const bf16*>(p.d_o) + base;
  bf16* __restrict__ dQ = static_cast<bf16*>(p.dq) + base;

  const int kv_lim = kv_limit(p, b, n);
  const int q0 = qb * kBR;
  const int qw0 = q0 + w * 32;
  const int qi = qw0 + c;
  const int qr = min(qi, n - 1);
  const float cs = p.c;

  // Q (sign-flipped for a negative scale) and dO rows of this wave as B
  // fragments [qi][kd*16 + h*8 + e]; rows past n read row n-1 (never stored).
  bf16x8 qf[ND], gf[ND];
  {
    const uint32_t flip = p.q_neg ? 0x80008000u : 0u;
#pragma unroll
    for (int kd = 0; kd < ND; ++kd) {
      qf[kd] = as_bf16x8(ld16(Q + (size_t)qr * D + kd * 16 + h * 8) ^ flip);
      gf[kd] = as_bf16x8(ld16(dO + (size_t)qr * D + kd * 16 + h * 8));
    }
  }
  // D_i and L_i log2(e) of this lane's row, also written to the workspace
  // for the dK/dV kernel (which runs after this one).
  float dd, l2;
  bwd_row_terms<ND>(p, bh, qi, n, static_cast<const bf16*>(p.o_in) + base + (size_t)qr * D, gf,
                    p.lse[qrow0 + qr], h, dd, l2);

  // Keys of this lane's row: [band.lo(qi), band.hi(qi)); key tiles [tb, te) hold every key
  // some row of the workgroup sees, tiles [ju_lo, ju_hi) only keys that all
  // of them see; keys [wlo, whi) are the ones some row of this wave sees.
  const Band<CAUSAL> band = make_band<CAUSAL>(p, n, kv_lim);
  const int q_last = min(q0 + kBR, n) - 1;
  const int tb = band.lo(q0) / BC;
  const int te = (band.hi(q_last) + BC - 1) / BC;
  const int ju_lo = (band.lo(q_last) + BC - 1) / BC;
  const int ju_hi = band.hi(q0) / BC;
  const int wlo = band.lo(qw0);
  const int whi = band.hi(min(qw0 + 31, n - 1));

  f32x16 acc[NMB];
#pragma unroll
  for (int mb = 0; mb < NMB; ++mb) acc[mb] = f32x16{};

  u32x4 kreg[KUPT][4];
  u32x4 vreg[VCH];

  // Key rows at or past the key limit are read clamped to the last visible
  // row; their probabilities are masked to exactly 0.
  auto gload = [&](int j) FA_INLINE {
    const int kb0 = j * BC;
#pragma unroll
    for (int i = 0; i < KUPT; ++i) {
      const int u = tid + i * kThreads;
      if (KUN % kThreads == 0 || u < KUN) {
        const int kg = (u >> 2) % (BC / 4);
        const int dg = (u & 3) + 4 * (u / BC);
#pragma unroll
        for (int r = 0; r < 4; ++r)
          kreg[i][r] = ld16(K + (size_t)min(kb0 + kg * 4 + r, kv_lim - 1) * D + dg * 8);
      }
    }
#pragma unroll
    for (int i = 0; i < VCH; ++i) {
      const int ch = tid + i * kThreads;
      const int key = min(kb0 + ch / (D / 8), kv_lim - 1);
      vreg[i] = ld16(V + (size_t)key * D + (ch % (D / 8)) * 8);
    }
  };

  auto swrite = [&]() FA_INLINE {
#pragma unroll
    for (int i = 0; i < KUPT; ++i) {
      const int u = tid + i * kThreads;
      if (KUN % kThreads == 0 || u < KUN) {
        const int kg = (u >> 2) % (BC / 4);
        const int dg = (u & 3) + 4 * (u / BC);
#pragma unroll
        for (int r = 0; r < 4; ++r)
          *reinterpret_cast<u32x4*>(&sK[(kg * 4 + r) * KSTR + dg * 8]) = kreg[i][r];
#pragma unroll
        for (int e = 0; e < 8; ++e)
          *reinterpret_cast<u32x2*>(&sKt[(dg * 8 + e) * TSTR + kg * 4]) = column4(kreg[i], e);
      }
    }
#pragma unroll
    for (int i = 0; i < VCH; ++i) {
      const int ch = tid + i * kThreads;
      *reinterpret_cast<u32x4*>(&sV[(ch / (D / 8)) * KSTR + (ch % (D / 8)) * 8]) = vreg[i];
    }
  };

  // Step on key tile j (registers hold it); the loads of tile jn, the next
  // one (or j again at the end), go out before the compute.
  auto step = [&](int j, int jn, auto mask_tag) FA_INLINE {
    constexpr bool MASK = decltype(mask_tag)::value;
    __syncthreads();  // every wave is done reading the previous tile
    swrite();
    __syncthreads();
    gload(jn);

    const int kb0 = j * BC;
    if (MASK && (kb0 >= whi || kb0 + BC <= wlo)) return;  // no row of this wave sees it

    // S^T = K Q^T and dP^T = V dO^T (keys x queries).
    f32x16 sv[NKB], dp[NKB];
#pragma unroll
    for (int kb = 0; kb < NKB; ++kb) {
      sv[kb] = f32x16{};
      dp[kb] = f32x16{};
#pragma unroll
      for (int kd = 0; kd < ND; ++kd) {
        const bf16x8 ka = as_bf16x8(ld16(&sK[(kb * 32 + c) * KSTR + kd * 16 + h * 8]));
        const bf16x8 va = as_bf16x8(ld16(&sV[(kb * 32 + c) * KSTR + kd * 16 + h * 8]));
        sv[kb] = mma32(ka, qf[kd], sv[kb]);
        dp[kb] = mma32(va, gf[kd], dp[kb]);
      }
    }
    // P^T = exp2(S^T c - L log2 e), dS^T = P^T (dP^T - D), as bf16 B
    // fragments: chunk (kb, kc) holds keys kb*32 + kc*16 + {h*4 + 0..3,
    // 8 + h*4 + 0..3}.
    bf16x8 sf[NKB * 2];
    // Row bounds of masked tiles, recomputed per tile from an opaque copy
    // of the row index (so they need no registers across the sweep).
    int lo_i = 0, hi_i = 0;
    if (MASK) {
      int qv = qi;
      asm volatile("" : "+v"(qv));
      lo_i = band.lo(qv);
      hi_i = band.hi(qv);
    }
#pragma unroll
    for (int kb = 0; kb < NKB; ++kb) {
      float ds[16];
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        float pr = __builtin_amdgcn_exp2f(fmaf(sv[kb][r], cs, -l2));
        if (MASK) {
          const int key = kb0 + kb * 32 + (r >> 2) * 8 + h * 4 + (r & 3);
          const bool hidden = key < lo_i || key >= hi_i;
          pr = hidden ? 0.f : pr;
        }
        ds[r] = pr * (dp[kb][r] - dd);
      }
#pragma unroll
      for (int kc = 0; kc < 2; ++kc) {
        u32x4 u;
#pragma unroll
        for (int t = 0; t < 4; ++t) u[t] = pack_bf16x2(ds[kc * 8 + 2 * t], ds[kc * 8 + 2 * t + 1]);
        sf[kb * 2 + kc] = as_bf16x8(u);
      }
    }
    // dQ^T (d x queries) += K^T dS^T.
#pragma unroll
    for (int mb = 0; mb < NMB; ++mb) {
#pragma unroll
      for (int kk = 0; kk < NKB * 2; ++kk) {
        const bf16* row = &sKt[(mb * 32 + c) * TSTR + kk * 16 + h * 4];
        const u32x2 lo = ld8(row);
        const u32x2 hi = ld8(row + 8);
        acc[mb] = mma32(as_bf16x8(u32x4{lo[0], lo[1], hi[0], hi[1]}), sf[kk], acc[mb]);
      }
    }
  };

  auto sweep = [&](const auto& tiles) FA_INLINE {
    const int ns = tiles.count;
    // Steps [su0, su1) hold the tiles every row sees in full.
    const int su0 = WIN ? tiles.first_at_least(ju_lo) : 0;
    const int su1 = max(tiles.first_at_least(ju_hi), su0);
    auto next = [&](int m) FA_INLINE { return tiles.tile(min(m + 1, ns - 1)); };
    if (ns > 0) gload(tiles.tile(0));
    int m = 0;
#pragma unroll 1
    for (; m < su0; ++m) step(tiles.tile(m), next(m), std::true_type{});
#pragma unroll 1
    for (; m < su1; ++m) step(tiles.tile(m), next(m), std::false_type{});
#pragma unroll 1
    for (; m < ns; ++m) step(tiles.tile(m), next(m), std::true_type{});
  };
  if constexpr (SPARSE) {
    // The workgroup's rows lie in one block row of the mask.
    const int nl = stage_blocks(row_blocks(p, q0 / kBlock), sblk, tid, kThreads, p.nb);
    sweep(sparse_tiles<kBlock / BC>(sblk, nl, tb, te));
  } else {
    sweep(dense_tiles(tb, te));
  }

  // dQ = scale * (dS K): the scores used Q' = sign(scale) Q with |scale|, the
  // accumulated sum is dS K with the true dS, so the signed scale applies.
  if (qi < n) {
    const float sc = p.scale;
    bf16* row = dQ + (size_t)qi * D;
#pragma unroll
    for (int mb = 0; mb < NMB; ++mb)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        u32x2 u;
        u[0] = pack_bf16x2(acc[mb][g * 4 + 0] * sc, acc[mb][g * 4 + 1] * sc);
        u[1] = pack_bf16x2(acc[mb][g * 4 + 2] * sc, acc[mb][g * 4 + 3] * sc);
        *reinterpret_cast<u32x2*>(row + mb * 32 + g * 8 + h * 4) = u;
      }
  }
}

template <int D, int BC>
hipError_t launch_d(const Params& p, hipStream_t s) {
  const int t_r = (p.n + kBR - 1) / kBR;
  const long long total = (long long)t_r * p.batch * p.heads;
  dim3 grid((unsigned)total), block(kThreads);
  return dispatch_mask_win(p, [&](auto causal, auto sparse, auto win) {
    hipLaunchKernelGGL((bwd_dq_staged_kernel<D, BC, decltype(causal)::value,
                                             decltype(sparse)::value, decltype(win)::value>),
                       grid, block, 0, s, p);
    return hipGetLastError();
  });
}

}  // namespace

hipError_t launch_bwd_dq_bf16_staged(const Params& p, int d, hipStream_t s) {
  switch (d) {
    case 256: return launch_d<256, 32>(p, s);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace fa
