// Attention backward, dQ part, d = 256: query-outer, software-pipelined
// within each wave.
//
// dQ = scale * dS K with dS = P * (dP - D), dP = dO V^T, and P rebuilt from
// the saved row statistic, P_ij = exp(scale q_i.k_j - L_i) (page 1, "注意力
// 为什么受限于显存带宽：用算术强度与分块把 FlashAttention 推导清楚", section 八;
// page 2, "4. FlashAttention 深度剖析", 4.3.4).
//
// Layout as in fa_bwd_dq_bf16.hip: a workgroup owns 128 query rows (4 waves
// x 32), Q and dO rows are B operands held in VGPRs, each wave forms
// S^T = K Q^T and dP^T = V dO^T for a 32-key tile, and dS^T rounded to bf16
// is the B operand of dQ^T += K^T dS^T. At d = 256 the dQ accumulator (128
// registers) and the Q and dO fragments (128) leave room for one wave per
// SIMD only, so no other wave runs its softmax arithmetic while this one
// uses the matrix core. The wave overlaps the two itself: step m forms S^T
// and dP^T of tile m, then runs the dQ^T products of tile m-1 with P^T and
// dS^T of tile m computed in the slots between them. K of tile m-1 is then
// still needed in step m (its transposing reads), so K and V tiles go
// through three LDS stages, each holding the K and the V tile of one key
// tile, filled straight from HBM through buffer descriptors one tile ahead,
// with one barrier per step.
#include <type_traits>

#include "fa_device.h"

namespace fa {

namespace {

constexpr int kThreads = 256;
constexpr int kBR = 128;  // query rows per workgroup (4 waves x 32)
constexpr int kD = 256;
constexpr int kBC = 32;   // keys per tile

template <bool CAUSAL, bool SPARSE, bool WIN>
__global__ __launch_bounds__(kThreads, 1) void bwd_dq_d256_kernel(Params p) {
  constexpr int D = kD;
  constexpr int BC = kBC;
  constexpr int CH = D / 8;             // 16-byte chunks per row
  constexpr int ROWB = D * 2;           // bytes per row
  constexpr int TILE = BC * D;          // elements per K or V tile
  constexpr int TILEB = TILE * 2;       // bytes per K or V tile
  constexpr int LPW = TILEB / 1024 / 4; // 1 KB wave loads per tensor per wave
  constexpr int RPL = 1024 / ROWB;      // rows per 1 KB load
  constexpr int ND = D / 16;            // reduction steps of S^T and dP^T
  constexpr int NMB = D / 32;           // 32-row blocks of dQ^T
  constexpr int HB = 2;                 // block flip of the +8-row half (see toff)
  static_assert(LPW * 4 * 1024 == TILEB && RPL >= 1, "tile split");

  // Stage s: K tile at [0, TILE), V tile at [TILE, 2 TILE).
  __shared__ __attribute__((aligned(1024))) bf16 sS0[2 * TILE];
  __shared__ __attribute__((aligned(1024))) bf16 sS1[2 * TILE];
  __shared__ __attribute__((aligned(1024))) bf16 sS2[2 * TILE];
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
  // for the dK/dV kernel (which runs after this one).
  float dd, l2;
  bwd_row_terms<ND>(p, bh, qi, n, static_cast<const bf16*>(p.o_in) + base + (size_t)qr * D, gf,
                    p.lse[qrow0 + qr], h, dd, l2);
  {
    const uint32_t flip = p.q_neg ? 0x80008000u : 0u;
#pragma unroll
    for (int kd = 0; kd < ND; ++kd)
      qf[kd] = as_bf16x8(ld16(Q + (size_t)qr * D + kd * 16 + h * 8) ^ flip);
  }

  // Keys of this lane's row: [band.lo(qi), band.hi(qi)); key tiles [tb, te)
  // hold every key some row of the workgroup sees, tiles [ju_lo, ju_hi) only
  // keys that all of them see; keys [wlo, whi) are the ones some row of this
  // wave sees.
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

  // Tile loads: wave w fills rows [w*LPW*RPL, (w+1)*LPW*RPL) of the K and the
  // V tile of a stage; lane l of a 1 KB load writes physical chunk l % CH of
  // row l / CH, holding logical chunk (l % CH) ^ swizzle(row). The
  // descriptor's base is the tile's first row and its size stops at the key
  // limit, so rows at or past it are never read. Load i covers rows 2i past
  // load 0's, whose swizzles differ from load 0's by a constant XOR of the
  // chunk index (10 (i & 1) + 4 (i >> 1) for the K swizzle, 2i for the V
  // one), and the row step (1024 i bytes) sets bits that the base offset
  // leaves clear: one base register per tensor and an XOR per load stand for
  // a table of offsets (the registers matter in a kernel this size). The
  // base offsets themselves are rebuilt from the lane id per tile (a fresh
  // v_mbcnt pair the compiler cannot hoist), so nothing is held across the
  // sweep for them.
  static_assert(D == 256 && LPW == 4 && RPL == 2, "offset XORs below");
  auto issue = [&](int j, bf16* st) FA_INLINE {
    const int kb0 = j * BC;
    const int bytes = max(min(kv_lim - kb0, BC), 0) * ROWB;
    const auto rk = buffer_rsrc(K + (size_t)kb0 * D, bytes);
    const auto rv = buffer_rsrc(V + (size_t)kb0 * D, bytes);
    int lid;
    asm volatile("v_mbcnt_lo_u32_b32 %0, -1, 0\n\tv_mbcnt_hi_u32_b32 %0, -1, %0" : "=v"(lid));
    const int row = w * LPW * RPL + lid / CH;
    const int kb = (row * D + ((lid % CH) ^ swz_both<D>(row)) * 8) * 2;
    const int vb = (row * D + ((lid % CH) ^ swz_row<D>(row)) * 8) * 2;
#pragma unroll
    for (int i = 0; i < LPW; ++i) {
      const int ko = kb ^ (((10 * (i & 1) + 4 * (i >> 1)) << 4) | (i << 10));
      const int vo = vb ^ (((2 * i) << 4) | (i << 10));
      bload_lds16(rk, ko, st + (w * LPW + i) * RPL * D);
      bload_lds16(rv, vo, st + TILE + (w * LPW + i) * RPL * D);
    }
  };
  // Out-of-range lanes of a partial tile may leave their LDS bytes as they
  // were, so every stage starts as zeros (finite data under every masked
  // score), and the zeros land before any wave's first loads.
  {
    constexpr int NZ = 2 * TILEB / 16 / kThreads;
    static_assert(NZ * 16 * kThreads == 2 * TILEB, "zero fill");
#pragma unroll
    for (int t = 0; t < NZ; ++t) {
      const int e = (t * kThreads + tid) * 8;
      *reinterpret_cast<u32x4*>(sS0 + e) = u32x4{0u, 0u, 0u, 0u};
      *reinterpret_cast<u32x4*>(sS1 + e) = u32x4{0u, 0u, 0u, 0u};
      *reinterpret_cast<u32x4*>(sS2 + e) = u32x4{0u, 0u, 0u, 0u};
    }
    __syncthreads();
  }

  // Per-lane LDS element offsets within a tile, as in fa_bwd_dq_bf16.hip: row
  // reads of K and V at kbase ^ (kd << 4) and vbase ^ (kd << 4); transposing
  // reads of K at tbase ^ (mb << 5), the second read of a fragment (rows +8)
  // in block mb ^ HB.
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

  // S^T and dP^T of the tile in stage st, in VGPRs (asm products; the
  // compiler would give the builtins AGPR accumulators in a kernel this
  // size; the w forms, since some Q and dO fragments live in AGPRs and are
  // read back right before their products). A fragments are read two products ahead through a ring of three,
  // pinned by the sched_barrier fences; mfma_drain lets the last products
  // finish before their results are read.
  auto scores = [&](const bf16* st, f32x16& s, f32x16& g) FA_INLINE {
    const bf16* sk = st;
    const bf16* sv = st + TILE;
    bf16x8 ka[3], va[3];
    ka[0] = as_bf16x8(ld16(sk + koff(0)));
    va[0] = as_bf16x8(ld16(sv + voff(0)));
    ka[1] = as_bf16x8(ld16(sk + koff(1)));
    va[1] = as_bf16x8(ld16(sv + voff(1)));
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int kd = 0; kd < ND; ++kd) {
      if (kd + 2 < ND) {
        ka[(kd + 2) % 3] = as_bf16x8(ld16(sk + koff(kd + 2)));
        va[(kd + 2) % 3] = as_bf16x8(ld16(sv + voff(kd + 2)));
      }
      if (kd == 0) {
        s = mma32_v0w(ka[0], qf[0]);
        g = mma32_v0w(va[0], gf[0]);
      } else {
        s = mma32_vw(ka[kd % 3], qf[kd], s);
        g = mma32_vw(va[kd % 3], gf[kd], g);
      }
      __builtin_amdgcn_sched_barrier(0);
    }
    mfma_drain();
  };

  // Transposed K fragment for dQ^T block mb and key chunk kk (16 keys).
  auto rd_kt = [&](const bf16* sk, int k) FA_INLINE {
    const int mb = k % NMB, kk = k / NMB;
    const u32x2 lo = ds_read_tr16(sk + kk * 16 * D + toff(mb));
    const u32x2 hi = ds_read_tr16(sk + (kk * 16 + 8) * D + toff(mb ^ HB));
    return as_bf16x8(u32x4{lo[0], lo[1], hi[0], hi[1]});
  };

  // dQ^T += K^T dS^T for the tile whose K is in stage st and whose dS^T
  // fragments are sf: slot k = product (mb = k % 8, kk = k / 8), so the two
  // products of one accumulator are eight slots apart.
  auto dq_products = [&](const bf16* st, const bf16x8 (&sf)[2]) FA_INLINE {
#pragma unroll
    for (int k = 0; k < 2 * NMB; ++k)
      acc[k % NMB] = mma32(rd_kt(st, k), sf[k / NMB], acc[k % NMB]);
  };

  // P^T = exp2(S^T c - L log2 e) and dS^T = P^T (dP^T - D) of element r
  // (key kb0 + (r/4)*8 + h*4 + r%4 of this lane's row); masked keys get P = 0.
  auto ds_elem = [&](const f32x16& s, const f32x16& g, int r, int kb0, int lo_i, int hi_i,
                     auto mask_tag) FA_INLINE {
    constexpr bool MASK = decltype(mask_tag)::value;
    float x = s[r];
    if (MASK) {
      const int key = kb0 + (r >> 2) * 8 + h * 4 + (r & 3);
      x = (key < lo_i || key >= hi_i) ? kNegInf : x;
    }
    const float pr = __builtin_amdgcn_exp2f(fmaf(x, cs, -l2));
    return pr * (g[r] - dd);
  };
  // The whole tile's dS^T as bf16 B fragments: chunk kc holds elements
  // kc*8 .. kc*8+7 (keys kc*16 + {h*4 + 0..3, 8 + h*4 + 0..3}).
  auto ds_tile = [&](const f32x16& s, const f32x16& g, int kb0, bf16x8 (&sf)[2],
                     auto mask_tag) FA_INLINE {
    int lo_i = 0, hi_i = 0;
    if (decltype(mask_tag)::value) {
      // Row bounds from an opaque copy of the row index (no registers held
      // across the sweep).
      int qv = qi;
      asm volatile("" : "+v"(qv));
      lo_i = band.lo(qv);
      hi_i = band.hi(qv);
    }
#pragma unroll
    for (int kc = 0; kc < 2; ++kc) {
      u32x4 u;
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        const int r = kc * 8 + 2 * t;
        u[t] = pack_bf16x2(ds_elem(s, g, r, kb0, lo_i, hi_i, mask_tag),
                           ds_elem(s, g, r + 1, kb0, lo_i, hi_i, mask_tag));
      }
      sf[kc] = as_bf16x8(u);
    }
  };

  // The hot form of phase two (unmasked tile, previous tile pending): the dQ^T
  // products of the previous tile, each slot carrying one element of this
  // tile's dS^T (its transposed K fragment read two slots ahead, fenced).
  auto dq_with_ds = [&](const bf16* prev, const bf16x8 (&sfp)[2], const f32x16& s,
                        const f32x16& g, bf16x8 (&sfn)[2]) FA_INLINE {
    constexpr int NS = 2 * NMB;
    bf16x8 fr[3];
    fr[0] = rd_kt(prev, 0);
    fr[1] = rd_kt(prev, 1);
    u32x4 pu[2];
    float dlo = 0.f;
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int k = 0; k < NS; ++k) {
      if (k + 2 < NS) fr[(k + 2) % 3] = rd_kt(prev, k + 2);
      acc[k % NMB] = mma32(fr[k % 3], sfp[k / NMB], acc[k % NMB]);
      const float x = ds_elem(s, g, k, 0, 0, 0, std::false_type{});
      if (k & 1) {
        pu[k >> 3][(k & 7) >> 1] = pack_bf16x2(dlo, x);
        // Pinned to this slot: the fragments are only read in the next
        // step, and the compiler would otherwise sink their arithmetic
        // there, out of the slots it is meant to fill.
        asm volatile("" : "+v"(pu[k >> 3][(k & 7) >> 1]));
      } else {
        dlo = x;
      }
      __builtin_amdgcn_sched_barrier(0);
    }
    sfn[0] = as_bf16x8(pu[0]);
    sfn[1] = as_bf16x8(pu[1]);
  };

  // Step m on tile j = tiles.tile(m): stage cur holds tile m (its loads were
  // issued one step earlier), prev tile m-1, and tile m+1 is loaded into nxt,
  // which held tile m-2 (last read in step m-1, before this step's barrier).
  // Each wave waits for its own loads of tile m, then the barrier makes every
  // wave's loads visible. `pend` says whether the wave owes the dQ^T products
  // of tile m-1 (fragments in sfp); a wave none of whose rows sees a masked
  // tile skips its products.
  bool pend = false;
  bf16x8 sfp[2];
  auto sweep = [&](const auto& tiles) FA_INLINE {
    const int ns = tiles.count;
    // Steps [su0, su1) hold the tiles every row sees in full.
    const int su0 = WIN ? tiles.first_at_least(ju_lo) : 0;
    const int su1 = max(tiles.first_at_least(ju_hi), su0);
    auto open = [&](int m, bf16* nxt) FA_INLINE {
      wait_global_loads();
      __syncthreads();
      if (m + 1 < ns) issue(tiles.tile(m + 1), nxt);
    };
    // General step: any mask, any pending state.
    auto gstep = [&](int m, bf16* cur, bf16* prev, bf16* nxt) FA_INLINE {
      open(m, nxt);
      const int kb0 = tiles.tile(m) * BC;
      const bool full = m >= su0 && m < su1;  // unmasked tile
      const bool need = full || !(kb0 >= whi || kb0 + BC <= wlo);
      f32x16 s, g;
      if (need) scores(cur, s, g);
      if (pend) dq_products(prev, sfp);
      if (need) {
        if (full) ds_tile(s, g, kb0, sfp, std::false_type{});
        else ds_tile(s, g, kb0, sfp, std::true_type{});
      }
      pend = need;
    };
    // Hot step: unmasked tile, previous tile pending (every step after the
    // first unmasked one). One straight path, so the accumulators never
    // cross a control-flow merge, which would cost a copy of all of them.
    auto hstep = [&](int m, bf16* cur, bf16* prev, bf16* nxt) FA_INLINE {
      open(m, nxt);
      f32x16 s, g;
      scores(cur, s, g);
      bf16x8 sfn[2];
      dq_with_ds(prev, sfp, s, g, sfn);
      sfp[0] = sfn[0];
      sfp[1] = sfn[1];
    };
    // Steps run in groups of three from a multiple of three, so each of the
    // three stage assignments has its own code: general steps up to the
    // first multiple of three past su0, hot groups while they lie below su1,
    // then general steps to the end.
    const int hb = min(ns, (su0 + 3) / 3 * 3);
    if (ns > 0) issue(tiles.tile(0), sS0);
    int m = 0;
    for (; m < hb; m += 3) {
      gstep(m, sS0, sS2, sS1);
      if (m + 1 >= hb) { m += 1; break; }
      gstep(m + 1, sS1, sS0, sS2);
      if (m + 2 >= hb) { m += 2; break; }
      gstep(m + 2, sS2, sS1, sS0);
    }
    if (m == hb && hb % 3 == 0) {
      for (; m + 3 <= su1; m += 3) {
        hstep(m, sS0, sS2, sS1);
        hstep(m + 1, sS1, sS0, sS2);
        hstep(m + 2, sS2, sS1, sS0);
      }
    }
    // m is a multiple of three here unless the first loop stopped at ns.
    for (; m < ns; m += 3) {
      gstep(m, sS0, sS2, sS1);
      if (m + 1 >= ns) break;
      gstep(m + 1, sS1, sS0, sS2);
      if (m + 2 >= ns) break;
      gstep(m + 2, sS2, sS1, sS0);
    }
    // The last tile's products (its K is still in its stage; nothing is
    // loaded any more).
    if (pend) {
      const int last = (ns - 1) % 3;
      if (last == 0) dq_products(sS0, sfp);
      else if (last == 1) dq_products(sS1, sfp);
      else dq_products(sS2, sfp);
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

}  // namespace

hipError_t launch_bwd_dq_bf16_d256(const Params& p, int d, hipStream_t s) {
  if (d != kD) return hipErrorInvalidValue;
  const int t_r = (p.n + kBR - 1) / kBR;
  const long long total = (long long)t_r * p.batch * p.heads;
  dim3 grid((unsigned)total), block(kThreads);
  return dispatch_mask_win(p, [&](auto causal, auto sparse, auto win) {
    hipLaunchKernelGGL((bwd_dq_d256_kernel<decltype(causal)::value, decltype(sparse)::value,
                                           decltype(win)::value>),
                       grid, block, 0, s, p);
    return hipGetLastError();
  });
}

}  // namespace fa
