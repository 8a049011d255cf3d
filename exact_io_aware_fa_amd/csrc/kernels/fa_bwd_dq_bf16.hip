// Attention backward, dQ part: bf16 in/out, fp32 accumulate, for gfx950
// (d = 64 and 128; d = 256 uses fa_bwd_dq_d256.hip).
//
// dQ = scale * dS K with dS = P * (dP - D), dP = dO V^T, and P rebuilt from
// the saved row statistic, P_ij = exp(scale q_i.k_j - L_i) (page 1, "注意力
// 为什么受限于显存带宽：用算术强度与分块把 FlashAttention 推导清楚", section 八;
// page 2, "4. FlashAttention 深度剖析", 4.3.4; the gradient formula itself is
// ordinary softmax calculus, the pages print none).
//
// This kernel is query-outer, like the forward: a workgroup owns 128 query
// rows (4 wave64s x 32) and sweeps the key/value tiles, so each dQ row is
// accumulated in registers by exactly one wave and written once -- no atomics
// and no dQ workspace. S and dP are recomputed here (the dK/dV kernel computes
// them too); the extra matrix work is cheaper on this GPU than adding dQ
// partial sums with device-wide float atomics, which are performed past the
// per-XCD L2 caches.
//
// Layout: each wave computes S^T = K Q^T and dP^T = V dO^T on the 32x32x16
// bf16 MFMA with Q and dO rows held in VGPRs as B operands, so a lane owns one
// query row and 16 keys of every 32-key block; L_i and D_i are per-lane
// constants. dS^T rounded to bf16 is already the B operand of
// dQ^T += K^T dS^T. K and V tiles go from HBM straight into LDS through
// buffer descriptors, in two stages (one barrier per tile). K is stored with
// a swizzle that serves both its row reads (A operand of S^T) and the
// transposing reads (ds_read_b64_tr_b16) that yield the K^T operand; V with
// the row-read swizzle. Two workgroups share each compute unit, so one wave's
// softmax arithmetic overlaps the other's matrix work.
#include <type_traits>

#include "fa_device.h"

namespace fa {

namespace {

constexpr int kThreads = 256;
constexpr int kBR = 128;  // query rows per workgroup (4 waves x 32)

template <int D, int BC, bool CAUSAL, bool SPARSE, bool WIN>
__global__ __launch_bounds__(kThreads, 2) void bwd_dq_kernel(Params p) {
  constexpr int CH = D / 8;             // 16-byte chunks per row
  constexpr int ROWB = D * 2;           // bytes per row
  constexpr int TILEB = BC * ROWB;      // bytes per K or V tile
  constexpr int LPW = TILEB / 1024 / 4; // 1 KB wave loads per tensor per wave
  constexpr int RPL = 1024 / ROWB;      // rows per 1 KB load
  constexpr int ND = D / 16;            // reduction steps of S^T and dP^T
  constexpr int NMB = D / 32;           // 32-row blocks of dQ^T
  constexpr int NKB = BC / 32;          // 32-key blocks of S^T
  constexpr int HB = D >= 128 ? 2 : 1;  // block flip of the +8-row half (see toff)
  static_assert(LPW * 4 * 1024 == TILEB && RPL >= 1, "tile split");
  static_assert(BC % 32 == 0 && D % 32 == 0, "tile shape");

  __shared__ __attribute__((aligned(1024))) bf16 sK0[BC * D];
  __shared__ __attribute__((aligned(1024))) bf16 sK1[BC * D];
  __shared__ __attribute__((aligned(1024))) bf16 sV0[BC * D];
  __shared__ __attribute__((aligned(1024))) bf16 sV1[BC * D];
  __shared__ int sblk[SPARSE ? kMaxBlocks : 1];

  const int tid = threadIdx.x;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
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
#pragma unroll
  for (int kd = 0; kd < ND; ++kd) gf[kd] = as_bf16x8(ld16(dO + (size_t)qr * D + kd * 16 + h * 8));
  // D_i and L_i log2(e) of this lane's row, also written to the workspace
  // for the dK/dV kernel (which runs after this one); formed before the Q
  // fragments are loaded, so the O row and Q never occupy registers at once.
  float dd, l2;
  bwd_row_terms<ND>(p, bh, qi, n, static_cast<const bf16*>(p.o_in) + base + (size_t)qr * D, gf,
                    p.lse[qrow0 + qr], h, dd, l2);
  {
    const uint32_t flip = p.q_neg ? 0x80008000u : 0u;
#pragma unroll
    for (int kd = 0; kd < ND; ++kd)
      qf[kd] = as_bf16x8(ld16(Q + (size_t)qr * D + kd * 16 + h * 8) ^ flip);
  }

  // Keys of this lane's row: [band.lo(qi), band.hi(qi)); key tiles [tb, te) hold every key
  // some row of the workgroup sees, tiles [ju_lo, ju_hi) only keys that all
  // of them see (the bounds are non-decreasing in the row); keys
  // [wlo, whi) are the ones some row of this wave sees.
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

  // Tile loads, as in the forward: wave w fills rows [w*LPW*RPL,
  // (w+1)*LPW*RPL); lane l of a 1 KB load writes physical chunk l % CH of
  // row l / CH, holding logical chunk (l % CH) ^ swizzle(row). The
  // descriptor's base is the tile's first row and its size stops at the key
  // limit, so rows at or past it are never read.
  int ld_koff[LPW], ld_voff[LPW];
#pragma unroll
  for (int i = 0; i < LPW; ++i) {
    const int row = (w * LPW + i) * RPL + lane / CH;
    ld_koff[i] = (row * D + ((lane % CH) ^ swz_both<D>(row)) * 8) * 2;
    ld_voff[i] = (row * D + ((lane % CH) ^ swz_row<D>(row)) * 8) * 2;
  }
  auto issue = [&](int j, bf16* dk, bf16* dv) FA_INLINE {
    const int kb0 = j * BC;
    const int bytes = max(min(kv_lim - kb0, BC), 0) * ROWB;
    const auto rk = buffer_rsrc(K + (size_t)kb0 * D, bytes);
    const auto rv = buffer_rsrc(V + (size_t)kb0 * D, bytes);
#pragma unroll
    for (int i = 0; i < LPW; ++i) {
      bload_lds16(rk, ld_koff[i], dk + (w * LPW + i) * RPL * D);
      bload_lds16(rv, ld_voff[i], dv + (w * LPW + i) * RPL * D);
    }
  };
  // Out-of-range lanes of a partial tile may leave their LDS bytes as they
  // were, so both stages start as zeros (finite data under every masked
  // score), and the zeros land before any wave's first loads.
  {
    constexpr int NZ = TILEB / 16 / kThreads;
    static_assert(NZ * 16 * kThreads == TILEB, "zero fill");
#pragma unroll
    for (int t = 0; t < NZ; ++t) {
      const int e = (t * kThreads + tid) * 8;
      *reinterpret_cast<u32x4*>(sK0 + e) = u32x4{0u, 0u, 0u, 0u};
      *reinterpret_cast<u32x4*>(sK1 + e) = u32x4{0u, 0u, 0u, 0u};
      *reinterpret_cast<u32x4*>(sV0 + e) = u32x4{0u, 0u, 0u, 0u};
      *reinterpret_cast<u32x4*>(sV1 + e) = u32x4{0u, 0u, 0u, 0u};
    }
    __syncthreads();
  }

  // Per-lane LDS element offsets (tile-invariant). Row reads of K and V: row
  // c of a 32-row block, logical chunk kd*2 + h, i.e. kbase ^ (kd << 4) and
  // vbase ^ (kd << 4). Transposing reads of K: row h*4 + (c%16)/4 of a 16-row
  // block, column mb*32 + 16*(c/16) + 4*(c%4), i.e. tbase ^ (mb << 5); the
  // second read of a fragment (rows +8) lands in block mb ^ HB. (The
  // swizzled chunk bits lie below the row's, so one base register and an
  // XOR per read replace a table of offsets: the registers this saves are
  // what keeps the sweep loops free of spills.)
  const int kbase = c * D + ((h ^ swz_both<D>(c)) << 3);
  const int vbase = c * D + ((h ^ swz_row<D>(c)) << 3);
  int tbase;
  {
    const int trow = h * 4 + ((c & 15) >> 2);
    const int tcol = 16 * (c >> 4) + 4 * (c & 3);
    tbase = trow * D + ((((tcol >> 3) ^ swz_both<D>(trow)) << 3) | (tcol & 7));
  }
  auto koff = [&](int kd) FA_INLINE { return kbase ^ (kd << 4); };
  auto voff = [&](int kd) FA_INLINE { return vbase ^ (kd << 4); };
  auto toff = [&](int mb) FA_INLINE { return tbase ^ (mb << 5); };

  // One key tile: S^T = K Q^T and dP^T = V dO^T (keys x queries), then
  // P^T = exp2(S^T c - L log2 e), dS^T = P^T (dP^T - D) as bf16 B fragments
  // (chunk (kb, kc) holds keys kb*32 + kc*16 + {h*4 + 0..3, 8 + h*4 + 0..3}),
  // then dQ^T += K^T dS^T.
  auto compute = [&](int j, const bf16* sk, const bf16* sv, auto mask_tag) FA_INLINE {
    constexpr bool MASK = decltype(mask_tag)::value;
    const int kb0 = j * BC;
    f32x16 s[NKB], g[NKB];
#pragma unroll
    for (int kb = 0; kb < NKB; ++kb) {
      s[kb] = f32x16{};
      g[kb] = f32x16{};
#pragma unroll
      for (int kd = 0; kd < ND; ++kd) {
        s[kb] = mma32(as_bf16x8(ld16(sk + kb * 32 * D + koff(kd))), qf[kd], s[kb]);
        g[kb] = mma32(as_bf16x8(ld16(sv + kb * 32 * D + voff(kd))), gf[kd], g[kb]);
      }
    }
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
        float x = s[kb][r];
        if (MASK) {
          const int key = kb0 + kb * 32 + (r >> 2) * 8 + h * 4 + (r & 3);
          const bool hidden = key < lo_i || key >= hi_i;
          x = hidden ? kNegInf : x;
        }
        const float pr = __builtin_amdgcn_exp2f(fmaf(x, cs, -l2));
        ds[r] = pr * (g[kb][r] - dd);
      }
#pragma unroll
      for (int kc = 0; kc < 2; ++kc) {
        u32x4 u;
#pragma unroll
        for (int t = 0; t < 4; ++t) u[t] = pack_bf16x2(ds[kc * 8 + 2 * t], ds[kc * 8 + 2 * t + 1]);
        sf[kb * 2 + kc] = as_bf16x8(u);
      }
    }
#pragma unroll
    for (int mb = 0; mb < NMB; ++mb)
#pragma unroll
      for (int kk = 0; kk < NKB * 2; ++kk) {
        const u32x2 lo = ds_read_tr16(sk + kk * 16 * D + toff(mb));
        const u32x2 hi = ds_read_tr16(sk + (kk * 16 + 8) * D + toff(mb ^ HB));
        acc[mb] = mma32(as_bf16x8(u32x4{lo[0], lo[1], hi[0], hi[1]}), sf[kk], acc[mb]);
      }
  };

  // Two LDS stages, one barrier per tile (as in the forward): at the top of
  // step m this wave waits for its own loads of the step's tile, the barrier
  // makes every wave's loads visible and guarantees every wave has finished
  // step m-1, whose stage is then refilled with the next tile. A wave none of
  // whose rows sees a masked tile skips it.
  auto sweep = [&](const auto& tiles) FA_INLINE {
    const int ns = tiles.count;
    // Steps [su0, su1) hold the tiles every row sees in full.
    const int su0 = WIN ? tiles.first_at_least(ju_lo) : 0;
    const int su1 = max(tiles.first_at_least(ju_hi), su0);
    auto iter = [&](int m, const bf16* sk, const bf16* sv, bf16* nk, bf16* nv,
                    auto mask_tag) FA_INLINE {
      constexpr bool MASK = decltype(mask_tag)::value;
      const int j = tiles.tile(m);
      wait_global_loads();
      __syncthreads();
      if (m + 1 < ns) issue(tiles.tile(m + 1), nk, nv);
      if (MASK && (j * BC >= whi || j * BC + BC <= wlo)) return;
      compute(j, sk, sv, mask_tag);
    };
    auto gen = [&](int m, const bf16* sk, const bf16* sv, bf16* nk, bf16* nv) FA_INLINE {
      if (m >= su0 && m < su1) iter(m, sk, sv, nk, nv, std::false_type{});
      else iter(m, sk, sv, nk, nv, std::true_type{});
    };
    if (ns > 0) issue(tiles.tile(0), sK0, sV0);
    // Whole pairs before the unmasked steps, unmasked pairs, then the rest
    // (a last single step only in the final loop).
    int m = 0;
    for (; m < su0 && m + 1 < ns; m += 2) {
      gen(m, sK0, sV0, sK1, sV1);
      gen(m + 1, sK1, sV1, sK0, sV0);
    }
    for (; m + 1 < su1; m += 2) {
      iter(m, sK0, sV0, sK1, sV1, std::false_type{});
      iter(m + 1, sK1, sV1, sK0, sV0, std::false_type{});
    }
    for (; m < ns; m += 2) {
      gen(m, sK0, sV0, sK1, sV1);
      if (m + 1 >= ns) break;
      gen(m + 1, sK1, sV1, sK0, sV0);
    }
  };
  if constexpr (SPARSE) {
    // The workgroup's 128 rows are one block row of the mask.
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
      for (int gi = 0; gi < 4; ++gi) {
        u32x2 u;
        u[0] = pack_bf16x2(acc[mb][gi * 4 + 0] * sc, acc[mb][gi * 4 + 1] * sc);
        u[1] = pack_bf16x2(acc[mb][gi * 4 + 2] * sc, acc[mb][gi * 4 + 3] * sc);
        *reinterpret_cast<u32x2*>(row + mb * 32 + gi * 8 + h * 4) = u;
      }
  }
}

template <int D, int BC>
hipError_t launch_d(const Params& p, hipStream_t s) {
  const int t_r = (p.n + kBR - 1) / kBR;
  const long long total = (long long)t_r * p.batch * p.heads;
  dim3 grid((unsigned)total), block(kThreads);
  return dispatch_mask_win(p, [&](auto causal, auto sparse, auto win) {
    hipLaunchKernelGGL((bwd_dq_kernel<D, BC, decltype(causal)::value, decltype(sparse)::value,
                                      decltype(win)::value>),
                       grid, block, 0, s, p);
    return hipGetLastError();
  });
}

}  // namespace

hipError_t launch_bwd_dq_bf16(const Params& p, int d, hipStream_t s) {
  switch (d) {
    case 64: return launch_d<64, 64>(p, s);
    case 128: return launch_d<128, 64>(p, s);
    case 256: return launch_bwd_dq_bf16_d256(p, d, s);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace fa
