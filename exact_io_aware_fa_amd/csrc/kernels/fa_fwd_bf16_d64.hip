// Fused attention forward, bf16, variant for d = 64.
//
// Same method, tile loads and wave layout as fa_fwd_bf16.hip (page 2, "4.
// FlashAttention 深度剖析", 4.3.2; page 1, "注意力为什么受限于显存带宽：用算术强度
// 与分块把 FlashAttention 推导清楚", section 六): S^T = K Q^T on the 32x32x16
// bf16 MFMA with Q in VGPRs, P kept in registers as the B operand of
// O^T += V^T P^T, K/V tiles loaded straight into swizzled LDS. The difference
// is the schedule: a workgroup is 4 waves (128 query rows), two workgroups
// share a compute unit, and every wave runs both the matrix products and the
// softmax of each tile. At d = 64 the softmax arithmetic of a tile outweighs
// its matrix work, so letting both waves of a SIMD do vector work at once
// beats the ping-pong schedule of the d = 128 kernel, where only one wave per
// SIMD does.
#include <type_traits>

#include "fa_device.h"

namespace fa {

namespace {

constexpr int kThreads = 256;
constexpr int kBR = 128;  // query rows per workgroup (4 waves x 32)
constexpr float kLazy = 64.f;  // reference lag bound (base 2), as for d = 128

// Exchange with the other 32-lane half of the wave (v_permlane32_swap): the
// two results hold the value of lane l % 32 and of lane l % 32 + 32 in some
// order, so their max (or sum) is the same on every lane.
__device__ __forceinline__ float halves_max(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x),
                                                  false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float halves_sum(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x),
                                                  false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

template <int D, int BC, int MINW, bool CAUSAL, bool SPARSE, bool WIN>
__global__ __launch_bounds__(kThreads, MINW) void fwd_bf16_d64_kernel(Params p) {
  constexpr int CH = D / 8;             // 16-byte chunks per row
  constexpr int ROWB = D * 2;           // bytes per row
  constexpr int TILEB = BC * ROWB;      // bytes per K or V tile
  constexpr int LPW = TILEB / 1024 / 4; // 1 KB wave loads per tensor per wave
  constexpr int RPL = 1024 / ROWB;      // rows per 1 KB load
  constexpr int ND = D / 16;            // reduction steps of S^T = K Q^T
  constexpr int NMB = D / 32;           // 32-row blocks of O^T
  constexpr int NKB = BC / 32;          // 32-key blocks of S^T
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
  bf16* __restrict__ O = static_cast<bf16*>(p.o) + base;

  const int kv_lim = kv_limit(p, b, n);
  const int q0 = qb * kBR;
  const int qw0 = q0 + w * 32;
  const int qi = qw0 + c;
  const float cs = p.c;

  // Q rows of this wave as B fragments: Q[qi][kd*16 + h*8 + e]. A negative
  // scale is applied by negating Q (exact); rows past n are zero.
  bf16x8 qf[ND];
  {
    const uint32_t flip = p.q_neg ? 0x80008000u : 0u;
    const int qr = min(qi, n - 1);
#pragma unroll
    for (int kd = 0; kd < ND; ++kd) {
      const u32x4 v = ld16(Q + (size_t)qr * D + kd * 16 + h * 8) ^ flip;
      qf[kd] = as_bf16x8(qi < n ? v : u32x4{0u, 0u, 0u, 0u});
    }
  }

  // Keys of this lane's row: [band.lo(qi), band.hi(qi)); key tiles [tb, te) hold every key
  // some row of the workgroup sees, tiles [ju_lo, ju_hi) only keys that all
  // of them see (the bounds are non-decreasing in the row); keys [wlo, whi)
  // are the ones some row of this wave sees.
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
  // Reference of the row's probabilities (P = exp2(s * cs - fref)), moved
  // only when the running max runs kLazy above it; the row-sum correction
  // lcorr and the rest of the lazy update are as in fa_fwd_bf16.hip.
  float fref = kNegInf;
  float lpart = 0.f;    // this half-wave's share of the running row sum
  float lcorr = 0.f;    // per tile: bf16(p_max) - p_max of its largest probability

  // Loads of a key (or value) tile into LDS. Wave w fills rows
  // [w * LPW * RPL, (w + 1) * LPW * RPL); lane l of a 1 KB load writes
  // physical chunk l % CH of row l / CH, which holds logical chunk
  // (l % CH) ^ swizzle(row). The loads go through a buffer descriptor whose
  // base is the tile's first row and whose size stops at the key limit, so
  // the per-lane byte offsets are tile-invariant and rows at or past the key
  // limit are never read (their scores are masked, they contribute 0).
  int ld_koff[LPW], ld_voff[LPW];
#pragma unroll
  for (int i = 0; i < LPW; ++i) {
    const int row = (w * LPW + i) * RPL + lane / CH;
    ld_koff[i] = (row * D + ((lane % CH) ^ swz_row<D>(row)) * 8) * 2;
    ld_voff[i] = (row * D + ((lane % CH) ^ swz_tr<D>(row)) * 8) * 2;
  }
  auto issue = [&](const bf16* src, const int (&off)[LPW], int j, bf16* dst) FA_INLINE {
    const int kb0 = j * BC;
    const auto r = buffer_rsrc(src + (size_t)kb0 * D, max(min(kv_lim - kb0, BC), 0) * ROWB);
#pragma unroll
    for (int i = 0; i < LPW; ++i) bload_lds16(r, off[i], dst + (w * LPW + i) * RPL * D);
  };
  // Out-of-range lanes of a partial tile may leave their LDS bytes as they
  // were, so both stages start as zeros: whatever a masked row holds is then
  // finite and its zero probability contributes exactly 0.
  {
    constexpr int NZ = 4 * TILEB / 16 / kThreads;
    static_assert(NZ * 16 * kThreads == 4 * TILEB, "zero fill");
#pragma unroll
    for (int t = 0; t < NZ; ++t) {
      const int idx = t * kThreads + tid;   // 16-byte chunk of the four tiles
      const int which = idx / (TILEB / 16);
      bf16* base = which == 0 ? sK0 : which == 1 ? sK1 : which == 2 ? sV0 : sV1;
      *reinterpret_cast<u32x4*>(base + (idx % (TILEB / 16)) * 8) = u32x4{0u, 0u, 0u, 0u};
    }
    __syncthreads();
  }

  // Per-lane LDS element offsets of the MFMA operand reads (tile-invariant):
  // K row c (rows kb*32 + c share the swizzle of c), logical chunk kd*2 + h;
  // V transposing reads at row h*4 + (c%16)/4 (+16 kk, +8), column
  // mb*32 + 16*(c/16) + 4*(c%4).
  int koff[ND], voff[NMB];
#pragma unroll
  for (int kd = 0; kd < ND; ++kd) koff[kd] = c * D + (((kd * 2 + h) ^ swz_row<D>(c)) << 3);
  {
    const int trow = h * 4 + ((c & 15) >> 2);
    const int tcol = 16 * (c >> 4) + 4 * (c & 3);
#pragma unroll
    for (int mb = 0; mb < NMB; ++mb) {
      const int col = mb * 32 + tcol;
      voff[mb] = trow * D + ((((col >> 3) ^ swz_tr<D>(trow))) << 3) + (col & 7);
    }
  }

  // S^T (keys x queries) = K Q^T for the tile in sk, raw dot products.
  auto scores = [&](const bf16* sk, f32x16 (&s)[NKB]) FA_INLINE {
#pragma unroll
    for (int kb = 0; kb < NKB; ++kb) {
      s[kb] = f32x16{};
#pragma unroll
      for (int kd = 0; kd < ND; ++kd) {
        const bf16x8 a = as_bf16x8(ld16(sk + kb * 32 * D + koff[kd]));
        s[kb] = mma32(a, qf[kd], s[kb]);
      }
    }
  };

  // Online-softmax update with the scores of tile j, then O^T += V^T P^T.
  auto softmax_pv = [&](int j, f32x16 (&s)[NKB], const bf16* sv, auto mask_tag) FA_INLINE {
    constexpr bool MASK = decltype(mask_tag)::value;
    const int kb0 = j * BC;
    if (MASK) {
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
      for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int key = kb0 + kb * 32 + (r >> 2) * 8 + h * 4 + (r & 3);
          const bool hidden = key < lo_i || key >= hi_i;
          s[kb][r] = hidden ? kNegInf : s[kb][r];
        }
    }
    // Lazy online update (see fa_fwd_bf16.hip): t = s * cs - fref, the
    // reference moving only when a row's max runs kLazy above it.
    float mt;  // the row's largest t (-inf if it sees no key of the tile)
    if (MASK) {
      // General tile: masked entries are -inf and the reference may be unset,
      // so the max is taken over the raw scores first.
      float mp[4] = {kNegInf, kNegInf, kNegInf, kNegInf};
#pragma unroll
      for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r) mp[r & 3] = fmaxf(mp[r & 3], s[kb][r]);
      const float mraw = halves_max(fmaxf(fmaxf(mp[0], mp[1]), fmaxf(mp[2], mp[3])));
      const float m2 = mraw * cs;  // -inf stays -inf (cs > 0)
      const bool move = m2 > fref + kLazy;  // also when the reference is unset
      if (__builtin_amdgcn_ballot_w64(move)) {
        const float alpha = move ? __builtin_amdgcn_exp2f(fref - m2) : 1.f;
#pragma unroll
        for (int mb = 0; mb < NMB; ++mb) acc[mb] *= alpha;
        lpart *= alpha;
        lcorr *= alpha;
        fref = move ? m2 : fref;
      }
      const float ref = fref == kNegInf ? 0.f : fref;
#pragma unroll
      for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r) s[kb][r] = fmaf(s[kb][r], cs, -ref);
      mt = fmaf(mraw, cs, -ref);
    } else {
      // Unmasked tile, every row's reference set (an earlier general step
      // covered the first tile each row sees): shift first, then the max.
#pragma unroll
      for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r) s[kb][r] = fmaf(s[kb][r], cs, -fref);
      float ma = fmaxf(s[0][0], s[0][1]), mc = fmaxf(s[0][2], s[0][3]);
#pragma unroll
      for (int i = 4; i < 16 * NKB; i += 4) {
        ma = fmaxf(fmaxf(ma, s[i / 16][i % 16]), s[i / 16][i % 16 + 1]);
        mc = fmaxf(fmaxf(mc, s[i / 16][i % 16 + 2]), s[i / 16][i % 16 + 3]);
      }
      mt = halves_max(fmaxf(ma, mc));
      if (__builtin_amdgcn_ballot_w64(mt > kLazy)) {
        const float delta = mt > kLazy ? mt : 0.f;  // per row: others move by 0
#pragma unroll
        for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
          for (int r = 0; r < 16; ++r) s[kb][r] -= delta;
        const float alpha = __builtin_amdgcn_exp2f(-delta);
#pragma unroll
        for (int mb = 0; mb < NMB; ++mb) acc[mb] *= alpha;
        lpart *= alpha;
        lcorr *= alpha;
        fref += delta;
        mt -= delta;
      }
    }
    float rp[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const float e = __builtin_amdgcn_exp2f(s[kb][r]);
        s[kb][r] = e;
        rp[r & 3] += e;
      }
    lpart += (rp[0] + rp[1]) + (rp[2] + rp[3]);
    {
      const float pm = __builtin_amdgcn_exp2f(mt);
      lcorr += __uint_as_float(pack_bf16x2(pm, 0.f) << 16) - pm;
    }

    // P^T as bf16 B fragments: chunk kk holds keys kk*16 + {h*4 + 0..3,
    // 8 + h*4 + 0..3}.
    bf16x8 pf[NKB * 2];
#pragma unroll
    for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
      for (int kc = 0; kc < 2; ++kc) {
        u32x4 u;
#pragma unroll
        for (int t = 0; t < 4; ++t)
          u[t] = pack_bf16x2(s[kb][kc * 8 + 2 * t], s[kb][kc * 8 + 2 * t + 1]);
        pf[kb * 2 + kc] = as_bf16x8(u);
      }

    // O^T (d x queries) += V^T P^T; the V^T fragment of (mb, kk) is two
    // transposing reads: keys kk*16 + h*4 + 0..3 and kk*16 + 8 + h*4 + 0..3
    // of column mb*32 + c.
#pragma unroll
    for (int mb = 0; mb < NMB; ++mb)
#pragma unroll
      for (int kk = 0; kk < NKB * 2; ++kk) {
        const u32x2 lo = ds_read_tr16(sv + kk * 16 * D + voff[mb]);
        const u32x2 hi = ds_read_tr16(sv + (kk * 16 + 8) * D + voff[mb]);
        acc[mb] = mma32(as_bf16x8(u32x4{lo[0], lo[1], hi[0], hi[1]}), pf[kk], acc[mb]);
      }
  };

  // Two LDS stages: at the top of step m this wave waits for its own loads
  // of the step's tile, then the barrier makes every wave's loads visible and
  // guarantees every wave has finished step m-1, whose stage is refilled
  // with the next tile right after. A wave none of whose rows sees a masked
  // tile skips it. Even steps use stage 0, odd steps stage 1.
  auto sweep = [&](const auto& tiles) FA_INLINE {
    const int ns = tiles.count;
    // Steps [su0, su1) hold tiles every row sees in full, after the first
    // such tile (which takes the general path: a row may see its first key
    // there, and the unmasked update needs every row's reference set).
    // (Clamped: with no such tile su0 would lie past the last step.)
    const int su0 = min((WIN ? tiles.first_at_least(ju_lo) : 0) + 1, ns);
    const int su1 = max(tiles.first_at_least(ju_hi), su0);
    auto iter = [&](int m, const bf16* sk, const bf16* sv, bf16* nk, bf16* nv,
                    auto mask_tag) FA_INLINE {
      constexpr bool MASK = decltype(mask_tag)::value;
      const int j = tiles.tile(m);
      wait_global_loads();
      __syncthreads();
      if (m + 1 < ns) {
        const int jn = tiles.tile(m + 1);
        issue(K, ld_koff, jn, nk);
        issue(V, ld_voff, jn, nv);
      }
      if (MASK && (j * BC >= whi || j * BC + BC <= wlo)) return;
      f32x16 sc[NKB];
      scores(sk, sc);
      softmax_pv(j, sc, sv, mask_tag);
    };
    auto gen = [&](int m, const bf16* sk, const bf16* sv, bf16* nk, bf16* nv) FA_INLINE {
      if (m >= su0 && m < su1) iter(m, sk, sv, nk, nv, std::false_type{});
      else iter(m, sk, sv, nk, nv, std::true_type{});
    };
    if (ns > 0) {
      const int j0 = tiles.tile(0);
      issue(K, ld_koff, j0, sK0);
      issue(V, ld_voff, j0, sV0);
    }
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

  // Epilogue: O = O~ / (l + lcorr) (bf16, round to nearest even),
  // L = ln 2 (fref + log2 l).
  const float l = halves_sum(lpart);
  if (qi < n) {
    const float inv = l > 0.f ? 1.f / (l + lcorr) : 0.f;
    bf16* orow = O + (size_t)qi * D;
#pragma unroll
    for (int mb = 0; mb < NMB; ++mb)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        u32x2 u;
        u[0] = pack_bf16x2(acc[mb][g * 4 + 0] * inv, acc[mb][g * 4 + 1] * inv);
        u[1] = pack_bf16x2(acc[mb][g * 4 + 2] * inv, acc[mb][g * 4 + 3] * inv);
        *reinterpret_cast<u32x2*>(orow + mb * 32 + g * 8 + h * 4) = u;
      }
    if (h == 0)
      p.lse[qrow0 + qi] = l > 0.f ? (fref + __log2f(l)) * kLn2 : kNegInf;
  }
}

template <int D, int BC, int MINW>
hipError_t launch_d(const Params& p, hipStream_t s) {
  const int t_r = (p.n + kBR - 1) / kBR;
  const long long total = (long long)t_r * p.batch * p.heads;
  dim3 grid((unsigned)total), block(kThreads);
  return dispatch_mask_win(p, [&](auto causal, auto sparse, auto win) {
    hipLaunchKernelGGL((fwd_bf16_d64_kernel<D, BC, MINW, decltype(causal)::value,
                                            decltype(sparse)::value, decltype(win)::value>),
                       grid, block, 0, s, p);
    return hipGetLastError();
  });
}

}  // namespace

hipError_t launch_fwd_bf16_d64(const Params& p, int d, hipStream_t s) {
  switch (d) {
    case 64: return launch_d<64, 64, 2>(p, s);
    // d = 128 with a block-sparse mask: 128-row workgroups lie in one block
    // row of the mask (the 256-row ping-pong workgroups would span two).
    case 128: return launch_d<128, 64, 2>(p, s);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace fa
