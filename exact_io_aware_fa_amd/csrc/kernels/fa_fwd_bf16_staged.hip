// Fused attention forward, bf16, register-staged variant (used for d = 256).
//
// Same method and wave layout as fa_fwd_bf16.hip (page 2, "4. FlashAttention
// 深度剖析", 4.3.2; page 1, "注意力为什么受限于显存带宽：用算术强度与分块把
// FlashAttention 推导清楚", section 六): 4 wave64s x 32 query rows, S^T = K Q^T
// on the 32x32x16 bf16 MFMA with Q in VGPRs, P kept in registers as the B
// operand of O^T += V^T P^T. The difference is how tiles reach LDS: each
// thread loads 16-byte chunks into registers and writes K row-major (rows
// padded by 16 bytes) and V transposed ([d][key], rows padded by 8 bytes,
// built with byte permutes), so every LDS operand read uses an immediate
// offset. At d = 256 the O accumulator (128 VGPRs) and Q fragments (64)
// leave no room for the per-lane address registers of the swizzled
// direct-to-LDS layout, and this variant is more than twice as fast there.
#include <type_traits>

#include "fa_device.h"

namespace fa {

namespace {

constexpr float kLazy = 64.f;  // reference lag bound (base 2), as for d = 128

constexpr int kThreads = 256;
constexpr int kBR = 128;  // query rows per workgroup (4 waves x 32)

template <int D, int BC, bool CAUSAL, bool SPARSE, bool WIN>
__global__ __launch_bounds__(kThreads, 2) void fwd_bf16_staged_kernel(Params p) {
  constexpr int KSTR = D + 8;    // K row stride in LDS (bf16 elements)
  constexpr int VSTR = BC + 4;   // V^T row stride in LDS (bf16 elements)
  constexpr int ND = D / 16;     // reduction steps of S^T = K Q^T
  constexpr int NMB = D / 32;    // 32-row blocks of O^T
  constexpr int NKB = BC / 32;   // 32-key blocks of S^T
  constexpr int KCH = BC * D / 8 / kThreads;  // 16-byte K chunks per thread
  constexpr int VUN = (BC / 4) * (D / 8);     // V units: 4 keys x 8 dims
  constexpr int VUPT = (VUN + kThreads - 1) / kThreads;
  static_assert(KCH * kThreads * 8 == BC * D, "K tile split");
  static_assert(BC % 32 == 0 && D % 32 == 0, "tile shape");

  __shared__ __attribute__((aligned(16))) bf16 sK[BC * KSTR];
  __shared__ __attribute__((aligned(16))) bf16 sVt[D * VSTR];
  __shared__ int sblk[SPARSE ? kMaxBlocks : 1];

  const int tid = threadIdx.x;
  const int w = tid >> 6;
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

  u32x4 kreg[KCH];
  u32x4 vreg[VUPT][4];

  // Fetch key/value tile j into registers. Rows at or past the key limit are
  // read clamped to the last visible row: their scores are masked to -inf,
  // so they contribute exactly 0, and padded rows are never read.
  auto gload = [&](int j) FA_INLINE {
    const int kb0 = j * BC;
#pragma unroll
    for (int i = 0; i < KCH; ++i) {
      const int ch = tid + i * kThreads;
      const int key = min(kb0 + ch / (D / 8), kv_lim - 1);
      kreg[i] = ld16(K + (size_t)key * D + (ch % (D / 8)) * 8);
    }
#pragma unroll
    for (int i = 0; i < VUPT; ++i) {
      const int u = tid + i * kThreads;
      if (VUN % kThreads == 0 || u < VUN) {
        const int kg = (u >> 2) % (BC / 4);
        const int dg = (u & 3) + 4 * (u / BC);
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int key = min(kb0 + kg * 4 + r, kv_lim - 1);
          vreg[i][r] = ld16(V + (size_t)key * D + dg * 8);
        }
      }
    }
  };

  auto swrite = [&]() FA_INLINE {
#pragma unroll
    for (int i = 0; i < KCH; ++i) {
      const int ch = tid + i * kThreads;
      const int key = ch / (D / 8);
      const int dc = ch % (D / 8);
      *reinterpret_cast<u32x4*>(&sK[key * KSTR + dc * 8]) = kreg[i];
    }
#pragma unroll
    for (int i = 0; i < VUPT; ++i) {
      const int u = tid + i * kThreads;
      if (VUN % kThreads == 0 || u < VUN) {
        const int kg = (u >> 2) % (BC / 4);
        const int dg = (u & 3) + 4 * (u / BC);
#pragma unroll
        for (int e = 0; e < 8; ++e)
          *reinterpret_cast<u32x2*>(&sVt[(dg * 8 + e) * VSTR + kg * 4]) =
              column4(vreg[i], e);
      }
    }
  };

  // Step on key tile j (registers hold it); the loads of tile jn, the next
  // one (or j again at the end), go out before the compute.
  auto step = [&](int j, int jn, auto mask_tag) FA_INLINE {
    constexpr bool MASK = decltype(mask_tag)::value;
    __syncthreads();  // every wave is done reading the previous tile
    swrite();
    __syncthreads();  // tile j is in LDS
    gload(jn);

    const int kb0 = j * BC;
    if (MASK && (kb0 >= whi || kb0 + BC <= wlo)) return;  // no row of this wave sees it

    // S^T (keys x queries) = K Q^T, raw dot products.
    f32x16 s[NKB];
#pragma unroll
    for (int kb = 0; kb < NKB; ++kb) {
      s[kb] = f32x16{};
#pragma unroll
      for (int kd = 0; kd < ND; ++kd) {
        const bf16x8 a = as_bf16x8(ld16(&sK[(kb * 32 + c) * KSTR + kd * 16 + h * 8]));
        s[kb] = mma32(a, qf[kd], s[kb]);
      }
    }
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
      float mraw = kNegInf;
#pragma unroll
      for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r) mraw = fmaxf(mraw, s[kb][r]);
      mraw = fmaxf(mraw, __shfl_xor(mraw, 32));
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
      mt = fmaxf(ma, mc);
      mt = fmaxf(mt, __shfl_xor(mt, 32));
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
    float rs = 0.f;
#pragma unroll
    for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const float e = __builtin_amdgcn_exp2f(s[kb][r]);
        s[kb][r] = e;
        rs += e;
      }
    lpart += rs;
    {
      const float pm = __builtin_amdgcn_exp2f(mt);
      lcorr += __uint_as_float(pack_bf16x2(pm, 0.f) << 16) - pm;
    }

    // P^T as bf16 B fragments: chunk (kb, kc) holds keys kb*32 + kc*16 +
    // {h*4 + 0..3, 8 + h*4 + 0..3}.
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

    // O^T (d x queries) += V^T P^T.
#pragma unroll
    for (int mb = 0; mb < NMB; ++mb)
#pragma unroll
      for (int kk = 0; kk < NKB * 2; ++kk) {
        const bf16* row = &sVt[(mb * 32 + c) * VSTR + kk * 16 + h * 4];
        const u32x2 lo = ld8(row);
        const u32x2 hi = ld8(row + 8);
        const u32x4 a = {lo[0], lo[1], hi[0], hi[1]};
        acc[mb] = mma32(as_bf16x8(a), pf[kk], acc[mb]);
      }
  };

  auto sweep = [&](const auto& tiles) FA_INLINE {
    const int ns = tiles.count;
    // Steps [su0, su1) hold tiles every row sees in full, after the first
    // such tile (which takes the general path: a row may see its first key
    // there, and the unmasked update needs every row's reference set).
    // (Clamped: with no such tile su0 would lie past the last step.)
    const int su0 = min((WIN ? tiles.first_at_least(ju_lo) : 0) + 1, ns);
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

  // Epilogue: O = O~ / (l + lcorr) (bf16, round to nearest even),
  // L = ln 2 (fref + log2 l).
  const float l = lpart + __shfl_xor(lpart, 32);
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

template <int D, int BC>
hipError_t launch_d(const Params& p, hipStream_t s) {
  const int t_r = (p.n + kBR - 1) / kBR;
  const long long total = (long long)t_r * p.batch * p.heads;
  dim3 grid((unsigned)total), block(kThreads);
  return dispatch_mask_win(p, [&](auto causal, auto sparse, auto win) {
    hipLaunchKernelGGL((fwd_bf16_staged_kernel<D, BC, decltype(causal)::value,
                                               decltype(sparse)::value, decltype(win)::value>),
                       grid, block, 0, s, p);
    return hipGetLastError();
  });
}

}  // namespace

hipError_t launch_fwd_bf16_staged(const Params& p, int d, hipStream_t s) {
  switch (d) {
    case 256: return launch_d<256, 32>(p, s);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace fa
