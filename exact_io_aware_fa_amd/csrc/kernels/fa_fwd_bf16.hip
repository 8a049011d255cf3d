// Fused attention forward, bf16 in/out, fp32 accumulate, for gfx950
// (d = 128 and 256; d = 64 and block-sparse d = 128 use fa_fwd_bf16_d64.hip).
//
// Method: the tiled forward of page 2 ("4. FlashAttention 深度剖析", 4.3.2)
// with the per-block (m, l, O) update of page 1 ("注意力为什么受限于显存带宽：
// 用算术强度与分块把 FlashAttention 推导清楚", section 六): query tiles outer,
// key/value tiles inner, normalisation deferred to the end, and the row
// statistic L = m + ln l stored for the backward pass. Causal key tiles that
// lie wholly above the diagonal are never visited (page 2 4.3.2's note; page 3
// "深入浅出 FlashAttention" 第八部分).
//
// Mapping onto CDNA4:
// * A workgroup is 8 wave64s (two per SIMD) and owns BR = 256 query rows;
//   each wave owns 32 of them for the whole key sweep (split over queries,
//   so no cross-wave reduction of m or l is ever needed).
// * Each wave keeps its Q rows in VGPRs as the B operand of the 32x32x16
//   bf16 MFMA and computes S^T = K Q^T, so a lane owns one query row and 16
//   keys of every 32-key block: the row max and row sum are in-lane, plus one
//   exchange between the two 32-lane halves (the max only; the sums are
//   combined once at the end).
// * The probabilities, rounded to bf16, are already laid out as the B
//   operand of O^T += V^T P^T, so P never leaves registers.
// * Ping-pong between the two waves of a SIMD: waves 0-3 (group A) and 4-7
//   (group B) alternate half-periods separated by workgroup barriers. In
//   each half-period one group runs its matrix phase (S of tile m and
//   O += P V of tile m-1) while the other runs its softmax phase (row max,
//   exp2, row sum, rescale and packing of tile m-1 or m). A wave issues
//   little vector work next to its own matrix products, but the other wave
//   on the SIMD can, so the two phases overlap on every SIMD.
// * K and V tiles go from HBM straight into LDS through buffer descriptors
//   whose size ends at the key limit (rows past it are never read),
//   row-major with an XOR swizzle of the 16-byte chunks, two stages each:
//   K of tile m+1 and V of tile m stream in during tile m's half-periods.
//   K is read row-wise (A operand of K Q^T); V is read with the transposing
//   LDS read, which yields the V^T operand directly. Both access patterns
//   hit every LDS bank once per 256 bytes.
// * exp2 with the log2(e) factor folded into the score scale; the max-shift
//   and scale are one FMA per score.
// * d = 256: a wave's O accumulator (128 registers) and Q fragments (64)
//   leave no room for a second wave on the SIMD, so the workgroup is 4
//   waves (128 rows), one per SIMD with up to 512 registers, each running
//   both phases of every step in turn (the schedule of group A below).
#include <type_traits>

#include "fa_device.h"

namespace fa {

namespace {

// The reference of a row's probabilities trails its running max by at most
// this much (base 2): probabilities stay in [0, 2^kLazy].
constexpr float kLazy = 64.f;

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

template <int D, int BC, bool CAUSAL, bool SPARSE, bool WIN, int NWAVES>
__global__ __launch_bounds__(NWAVES * 64, 1) void fwd_bf16_kernel(Params p) {
  // 8 waves: ping-pong between waves w and w + 4 (groups A and B); 4 waves:
  // every wave is in group A and runs both phases of each step.
  constexpr int kThreads = NWAVES * 64;
  constexpr int kBR = 32 * NWAVES;      // query rows per workgroup
  static_assert(NWAVES == 8 || NWAVES == 4, "workgroup shape");
  // A block-sparse mask needs the workgroup's rows in one block row.
  static_assert(!SPARSE || 32 * NWAVES == kBlock, "block-sparse workgroups are one block row");
  constexpr int CH = D / 8;             // 16-byte chunks per row
  constexpr int ROWB = D * 2;           // bytes per row
  constexpr int TILEB = BC * ROWB;      // bytes per K or V tile
  constexpr int NW = kThreads / 64;     // waves per workgroup
  constexpr int LPW = TILEB / 1024 / NW;  // 1 KB wave loads per tensor per wave
  constexpr int RPL = 1024 / ROWB;      // rows per 1 KB load
  constexpr int ND = D / 16;            // reduction steps of S^T = K Q^T
  constexpr int NMB = D / 32;           // 32-row blocks of O^T
  constexpr int NKB = BC / 32;          // 32-key blocks of S^T
  static_assert(LPW * NW * 1024 == TILEB && RPL >= 1, "tile split");
  static_assert(BC % 32 == 0 && D % 32 == 0, "tile shape");

  __shared__ __attribute__((aligned(1024))) bf16 sK0[BC * D];
  __shared__ __attribute__((aligned(1024))) bf16 sK1[BC * D];
  __shared__ __attribute__((aligned(1024))) bf16 sV0[BC * D];
  __shared__ __attribute__((aligned(1024))) bf16 sV1[BC * D];
  __shared__ int sblk[SPARSE ? kMaxBlocks : 1];

  const int tid = threadIdx.x;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int grp = NWAVES == 8 ? (w >> 2) : 0;  // 0: group A, 1: group B
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
  // Rows of wave w: the two waves of a SIMD (w and w + 4) take neighbouring
  // 32-row blocks, so both groups span the workgroup's 256 rows and reach
  // the causal diagonal at about the same step.
  const int qw0 = NWAVES == 8 ? q0 + 32 * (2 * (w & 3) + grp) : q0 + 32 * w;
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

  // Keys of this lane's row: [band.lo(qi), band.hi(qi)). Step m of the
  // sweep handles key tile tile_of(m): tb + m, or with a block mask the m-th
  // tile of the listed blocks of the workgroup's block row inside
  // [tb, te). This wave's rows need steps [s_first, s_last], and steps
  // [su_lo, su_hi) hold only keys every row of the wave sees (the bounds are
  // non-decreasing in the row, and so are the tiles of the steps); the
  // other steps of the wave are masked.
  const Band<CAUSAL> band = make_band<CAUSAL>(p, n, kv_lim);
  const int tb = band.lo(q0) / BC;
  const int te = (band.hi(min(q0 + kBR, n) - 1) + BC - 1) / BC;
  const int qw_last = min(qw0 + 31, n - 1);
  SparseTiles<kBlock / BC> st{};
  if constexpr (SPARSE) {
    const int nl = stage_blocks(row_blocks(p, q0 / kBlock), sblk, tid, kThreads, p.nb);
    st = sparse_tiles<kBlock / BC>(sblk, nl, tb, te);
  }
  auto tile_of = [&](int m) FA_INLINE {
    if constexpr (SPARSE) return st.tile(m);
    else return tb + m;
  };
  const int ntiles = SPARSE ? st.count : max(te - tb, 0);
  int s_first, s_last, su_lo, su_hi;
  if constexpr (SPARSE) {
    s_first = st.first_at_least(band.lo(qw0) / BC);
    s_last = st.first_at_least((band.hi(qw_last) + BC - 1) / BC) - 1;
    su_lo = st.first_at_least((band.lo(qw_last) + BC - 1) / BC);
    su_hi = st.first_at_least(band.hi(qw0) / BC);
  } else {
    s_first = band.lo(qw0) / BC - tb;
    s_last = (band.hi(qw_last) - 1) / BC - tb;
    su_lo = (band.lo(qw_last) + BC - 1) / BC - tb;
    su_hi = band.hi(qw0) / BC - tb;
  }

  f32x16 acc[NMB];
#pragma unroll
  for (int mb = 0; mb < NMB; ++mb) acc[mb] = f32x16{};
  // Reference of the row's probabilities, in scaled base-2 units (s * cs):
  // P = exp2(s * cs - fref). It is the exact running max when set, and is
  // only moved up (with a rescale of O~, l and lcorr) once the running max
  // runs more than kLazy above it, so probabilities lie in [0, 2^kLazy].
  float fref = kNegInf;
  float lpart = 0.f;    // this half-wave's share of the running row sum
  // Row-sum correction: for every tile, bf16(p_max) - p_max of the tile's
  // largest probability (the same in both halves of the wave).
  float lcorr = 0.f;
  f32x16 sc[NKB];       // scores of the tile between the two phases
  bf16x8 pf[NKB * 2];   // P^T fragments of the tile between the two phases
#pragma unroll
  for (int kk = 0; kk < NKB * 2; ++kk) pf[kk] = as_bf16x8(u32x4{0u, 0u, 0u, 0u});
  // 4 waves: the hot steps alternate between pf and pf2 (one holds P of the
  // previous tile for its P V product while the softmax fills the other).
  bf16x8 pf2[NWAVES == 4 ? NKB * 2 : 1];

  // Loads of a key (or value) tile into LDS. Wave w fills rows
  // [w * LPW * RPL, (w + 1) * LPW * RPL); lane l of a 1 KB load writes
  // physical chunk l % CH of row l / CH, which holds logical chunk
  // (l % CH) ^ swizzle(row). The descriptor's base is the tile's first row
  // and its size ends at the key limit, so the per-lane byte offsets are
  // tile-invariant and rows at or past the limit are never read.
  int ld_koff[LPW], ld_voff[LPW];
#pragma unroll
  for (int i = 0; i < LPW; ++i) {
    const int row = (w * LPW + i) * RPL + lane / CH;
    ld_koff[i] = (row * D + ((lane % CH) ^ swz_row<D>(row)) * 8) * 2;
    ld_voff[i] = (row * D + ((lane % CH) ^ swz_tr<D>(row)) * 8) * 2;
  }
  auto issue = [&](const bf16* src, const int (&off)[LPW], int j, bf16* dst) FA_INLINE {
    const int kb0 = tile_of(j) * BC;
    const auto r = buffer_rsrc(src + (size_t)kb0 * D, max(min(kv_lim - kb0, BC), 0) * ROWB);
#pragma unroll
    for (int i = 0; i < LPW; ++i) bload_lds16(r, off[i], dst + (w * LPW + i) * RPL * D);
  };
  // Out-of-range lanes of a partial tile may leave their LDS bytes as they
  // were, so all stages start as zeros: whatever a masked row holds is then
  // finite and its zero probability contributes exactly 0.
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

  // Per-lane LDS element offsets of the MFMA operand reads (tile-invariant):
  // K row c (rows kb*32 + c share the swizzle of c), logical chunk kd*2 + h;
  // V transposing reads at row h*4 + (c%16)/4 (+16 kk, +8), column
  // mb*32 + 16*(c/16) + 4*(c%4).
  // With 4 waves (d = 256: 16 + 8 offsets, and registers are scarce) each
  // is a base register XOR a per-index constant instead: the swizzled chunk
  // bits lie below the row's, so kd (mb) only flips bits 4.. (5..).
  constexpr bool XOFF = NWAVES == 4;
  int koff[XOFF ? 1 : ND], voff[XOFF ? 1 : NMB];
  int kbase = 0, vbase = 0;
  if constexpr (!XOFF) {
#pragma unroll
    for (int kd = 0; kd < ND; ++kd) koff[kd] = c * D + (((kd * 2 + h) ^ swz_row<D>(c)) << 3);
  }
  {
    const int trow = h * 4 + ((c & 15) >> 2);
    const int tcol = 16 * (c >> 4) + 4 * (c & 3);
    if constexpr (XOFF) {
      kbase = c * D + ((h ^ swz_row<D>(c)) << 3);
      vbase = trow * D + ((((tcol >> 3) ^ swz_tr<D>(trow)) << 3) | (tcol & 7));
    } else {
#pragma unroll
      for (int mb = 0; mb < NMB; ++mb) {
        const int col = mb * 32 + tcol;
        voff[mb] = trow * D + ((((col >> 3) ^ swz_tr<D>(trow))) << 3) + (col & 7);
      }
    }
  }
  auto ko = [&](int kd) FA_INLINE {
    if constexpr (XOFF) return kbase ^ (kd << 4);
    else return koff[kd];
  };
  auto vo = [&](int mb) FA_INLINE {
    if constexpr (XOFF) return vbase ^ (mb << 5);
    else return voff[mb];
  };

  // Matrix phase of step m: S^T of tile m (K in sk) into sc and
  // O^T += V^T P^T of tile m-1 (V in sv, P^T in pf), as a fixed sequence of
  // product slots: the S^T slots first (so the scores are ready early for a
  // softmax phase that follows at once), then the O^T slots (four
  // independent accumulators in turn). Each slot's A fragment is read PF
  // slots ahead (a ring of
  // PF + 1), and the sched_barrier fences keep the compiler from hoisting
  // every read to the top of the phase, which would exhaust the registers.
  constexpr int NPV = NMB * NKB * 2;  // O^T slots
  constexpr int PF = 6;               // read-ahead distance in slots
  constexpr int NS = NKB * ND;        // S^T slots
  auto rd_pv = [&](const bf16* sv, int k) FA_INLINE {
    const int mb = k % NMB, kk = k / NMB;
    const u32x2 lo = ds_read_tr16(sv + kk * 16 * D + vo(mb));
    const u32x2 hi = ds_read_tr16(sv + (kk * 16 + 8) * D + vo(mb));
    return as_bf16x8(u32x4{lo[0], lo[1], hi[0], hi[1]});
  };
  auto rd_s = [&](const bf16* sk, int k) FA_INLINE {
    const int kb = k % NKB, kd = k / NKB;
    return as_bf16x8(ld16(sk + kb * 32 * D + ko(kd)));
  };
  auto slots = [&](const bf16* sk, const bf16* sv, auto pv_tag, auto s_tag) FA_INLINE {
    constexpr bool PV = decltype(pv_tag)::value;
    constexpr bool SS = decltype(s_tag)::value;
    constexpr int K0 = SS ? 0 : NS;            // first slot
    constexpr int K1 = PV ? NS + NPV : NS;     // one past the last slot
    auto rd = [&](int k) FA_INLINE { return k < NS ? rd_s(sk, k) : rd_pv(sv, k - NS); };
    if (SS) {
#pragma unroll
      for (int kb = 0; kb < NKB; ++kb) sc[kb] = f32x16{};
    }
    bf16x8 fr[PF + 1];
#pragma unroll
    for (int k = K0; k < K0 + PF && k < K1; ++k) fr[k % (PF + 1)] = rd(k);
#pragma unroll
    for (int k = K0; k < K1; ++k) {
      if (k + PF < K1) fr[(k + PF) % (PF + 1)] = rd(k + PF);
      if (k < NS) {
        const int kb = k % NKB, kd = k / NKB;
        sc[kb] = mma32(fr[k % (PF + 1)], qf[kd], sc[kb]);
      } else {
        const int mb = (k - NS) % NMB, kk = (k - NS) / NMB;
        acc[mb] = mma32(fr[k % (PF + 1)], pf[kk], acc[mb]);
      }
      __builtin_amdgcn_sched_barrier(0);
    }
  };
  // The matrix phase always runs both products: at step 0 and after a
  // skipped tile P^T is zero (and the V stage holds finite data), so O~ is
  // unchanged; scores computed for a tile this wave will not use are
  // discarded.
  auto mfma_phase = [&](int m, const bf16* sk, const bf16* sv) FA_INLINE {
    (void)m;
    slots(sk, sv, std::true_type{}, std::true_type{});
  };

  // Softmax phase of tile j: online update of (m, l) with the scores in sc,
  // rescale of O~ (skipped, wave-uniformly, when no row max changed), and
  // P^T as bf16 B fragments in pf (chunk kk holds keys kk*16 + {h*4 + 0..3,
  // 8 + h*4 + 0..3}).
  auto apply_mask = [&](int j) FA_INLINE {
    const int kb0 = tile_of(j) * BC;
    // Row bounds, recomputed per masked tile from an opaque copy of the
    // row index (so they need no registers across the sweep).
    int qv = qi;
    asm volatile("" : "+v"(qv));
    const int lo_i = band.lo(qv), hi_i = band.hi(qv);
#pragma unroll
    for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int key = kb0 + kb * 32 + (r >> 2) * 8 + h * 4 + (r & 3);
        const bool hidden = key < lo_i || key >= hi_i;
        sc[kb][r] = hidden ? kNegInf : sc[kb][r];
      }
  };
  // The online update with a lazy reference (page 1 section 六's running
  // max is still formed every tile, but O~ and l are rescaled only when it
  // runs kLazy above the reference). Exactness of the result does not depend
  // on the reference; what matters for accuracy is that the weights the P V
  // product uses (bf16-rounded P) and the row sum it is normalised by agree.
  // l sums the fp32 P (so the LSE is that of the fp32 probabilities), and
  // lcorr adds, per tile, the rounding bf16(p) - p of the tile's largest
  // probability: a row dominated by one key is then normalised by exactly
  // the weight its product used. (With the exact max as reference that
  // weight is exactly 1 and needs no correction; with a lazy one it is
  // 2^delta, rounded.)
  auto finish_tile = [&](float mt, bf16x8 (&pout)[NKB * 2]) FA_INLINE {
    // sc holds t = s * cs - fref; mt is the row's largest t (-inf if none).
    float rp[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const float e = __builtin_amdgcn_exp2f(sc[kb][r]);
        sc[kb][r] = e;
        rp[r & 3] += e;
      }
    lpart += (rp[0] + rp[1]) + (rp[2] + rp[3]);
    // The tile's largest probability (exp2 of the same operand as its
    // element's) and its bf16 rounding error; an empty row adds 0 - 0.
    const float pm = __builtin_amdgcn_exp2f(mt);
    lcorr += __uint_as_float(pack_bf16x2(pm, 0.f) << 16) - pm;
#pragma unroll
    for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
      for (int kc = 0; kc < 2; ++kc) {
        u32x4 u;
#pragma unroll
        for (int t = 0; t < 4; ++t)
          u[t] = pack_bf16x2(sc[kb][kc * 8 + 2 * t], sc[kb][kc * 8 + 2 * t + 1]);
        pout[kb * 2 + kc] = as_bf16x8(u);
      }
    // Pin the results here: otherwise the compiler sinks the exponentials
    // and the packing past the next barrier, next to their use in the
    // matrix phase, where they would no longer overlap the other group's
    // matrix work.
#pragma unroll
    for (int kk = 0; kk < NKB * 2; ++kk) asm volatile("" : "+v"(pout[kk]));
    asm volatile("" : "+v"(lpart), "+v"(lcorr));
  };
  auto rescale = [&](float alpha) FA_INLINE {
#pragma unroll
    for (int q = 0; q < NMB; ++q) acc[q] *= alpha;
    lpart *= alpha;
    lcorr *= alpha;
  };
  // Unmasked tile whose rows all have a finite reference (every row has
  // seen a visible key in an earlier, general step): the scores are shifted
  // first, t = s * cs - fref, and the row max is taken over t (results of
  // arithmetic, so the max needs no NaN quieting of its inputs).
  auto softmax_hot = [&]() FA_INLINE {
#pragma unroll
    for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
      for (int r = 0; r < 16; ++r) sc[kb][r] = fmaf(sc[kb][r], cs, -fref);
    float ma = fmaxf(sc[0][0], sc[0][1]), mb = fmaxf(sc[0][2], sc[0][3]);
#pragma unroll
    for (int i = 4; i < 16 * NKB; i += 4) {
      ma = fmaxf(fmaxf(ma, sc[i / 16][i % 16]), sc[i / 16][i % 16 + 1]);
      mb = fmaxf(fmaxf(mb, sc[i / 16][i % 16 + 2]), sc[i / 16][i % 16 + 3]);
    }
    float mt = halves_max(fmaxf(ma, mb));
    if (__builtin_amdgcn_ballot_w64(mt > kLazy)) {
      // Move the reference of each row whose max ran kLazy ahead up to that
      // max (its largest t becomes exactly 0); the other rows move by 0, an
      // exact no-op, so every row's result depends on its own scores only.
      const float delta = mt > kLazy ? mt : 0.f;
#pragma unroll
      for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r) sc[kb][r] -= delta;
      rescale(__builtin_amdgcn_exp2f(-delta));
      fref += delta;
      mt -= delta;
    }
    finish_tile(mt, pf);
  };
  // General tile (masked entries -inf, references possibly unset): the max
  // is taken over the raw scores first, the reference is set (or moved) to
  // the running max when it is unset or runs kLazy ahead.
  auto softmax = [&]() FA_INLINE {
    float mp[4] = {kNegInf, kNegInf, kNegInf, kNegInf};
#pragma unroll
    for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
      for (int r = 0; r < 16; ++r) mp[r & 3] = fmaxf(mp[r & 3], sc[kb][r]);
    const float mraw = halves_max(fmaxf(fmaxf(mp[0], mp[1]), fmaxf(mp[2], mp[3])));
    const float m2 = mraw * cs;  // -inf stays -inf (cs > 0)
    const bool move = m2 > fref + kLazy;  // also when the reference is unset
    if (__builtin_amdgcn_ballot_w64(move)) {
      // Rows that move take their running max as the reference (an unset
      // one gives alpha = exp2(-inf) = 0, on sums that are 0); the others
      // keep theirs and are scaled by exactly 1.
      rescale(move ? __builtin_amdgcn_exp2f(fref - m2) : 1.f);
      fref = move ? m2 : fref;
    }
    // Rows without a visible key so far: every score is -inf, t = -inf.
    const float ref = fref == kNegInf ? 0.f : fref;
#pragma unroll
    for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
      for (int r = 0; r < 16; ++r) sc[kb][r] = fmaf(sc[kb][r], cs, -ref);
    finish_tile(fmaf(mraw, cs, -ref), pf);
  };
  // General softmax phase of step j: tiles this wave does not need (before
  // the first step, outside its rows' keys or past the last) leave P^T zero,
  // so the next matrix phase, which always runs both products, adds exactly
  // 0. Masking only edits the scores ahead of the common softmax body.
  auto valu_phase = [&](int j) FA_INLINE {
    if (j >= 0 && j < ntiles && j >= s_first && j <= s_last) {
      if (j < su_lo || j >= su_hi) apply_mask(j);
      softmax();
    } else {
#pragma unroll
      for (int kk = 0; kk < NKB * 2; ++kk) pf[kk] = as_bf16x8(u32x4{0u, 0u, 0u, 0u});
    }
  };

  // Step m covers two half-periods, each opening with a workgroup barrier.
  // At the first, K of tile m (stage m % 2) and V of tile m-1 (the other
  // stage) are resident; the loads of K of tile m+1 and V of tile m go into
  // the stages those tiles' predecessors held (last read in the previous
  // step's half-periods, which every wave has finished at this barrier).
  // Each wave waits for its own loads of a step before the next step's
  // first barrier. Group A: matrix phase m, then softmax phase m; group B:
  // softmax phase m-1, then matrix phase m. Each group runs its own loop;
  // both pass the same number of barriers.
  // Workgroup barriers that no instruction is scheduled across (the
  // compiler may otherwise move register-only work, such as softmax
  // arithmetic, over them into the other phase, which would undo the
  // ping-pong). The step-opening barrier is a full __syncthreads (it
  // publishes the tile loads each wave has waited for); the one between the
  // two phases of a step orders no memory, so it is a bare s_barrier and does
  // not wait for the loads still in flight.
  auto phase_barrier = [&]() FA_INLINE {
    __builtin_amdgcn_sched_barrier(0);
    __syncthreads();
    __builtin_amdgcn_sched_barrier(0);
  };
  // With 4 waves there is no partner group to keep in phase, and every
  // step must pass the same number of barriers in every wave (the hot step
  // below has no mid-step barrier), so it is left out.
  auto mid_barrier = [&]() FA_INLINE {
    if constexpr (NWAVES == 8) {
      __builtin_amdgcn_sched_barrier(0);
      __builtin_amdgcn_s_barrier();
      __builtin_amdgcn_sched_barrier(0);
    }
  };
  auto open_step = [&](int m, bf16* nk, bf16* nv) FA_INLINE {
    if (m > 0) wait_global_loads();
    phase_barrier();
    if (m + 1 < ntiles) issue(K, ld_koff, m + 1, nk);
    if (m < ntiles) issue(V, ld_voff, m, nv);
  };
  auto step_a = [&](int m, const bf16* sk, bf16* nk, bf16* nv, const bf16* sv) FA_INLINE {
    open_step(m, nk, nv);
    mfma_phase(m, sk, sv);
    mid_barrier();
    valu_phase(m);
  };
  auto step_b = [&](int m, const bf16* sk, bf16* nk, bf16* nv, const bf16* sv) FA_INLINE {
    open_step(m, nk, nv);
    valu_phase(m - 1);
    mid_barrier();
    mfma_phase(m, sk, sv);
  };
  // The same steps when both products run and the softmax is unmasked: one
  // straight path, so the accumulators never cross a control-flow merge
  // (which would cost register copies of all of them).
  auto hot_a = [&](int m, const bf16* sk, bf16* nk, bf16* nv, const bf16* sv) FA_INLINE {
    open_step(m, nk, nv);
    slots(sk, sv, std::true_type{}, std::true_type{});
    mid_barrier();
    softmax_hot();
  };
  auto hot_b = [&](int m, const bf16* sk, bf16* nk, bf16* nv, const bf16* sv) FA_INLINE {
    open_step(m, nk, nv);
    softmax_hot();
    mid_barrier();
    slots(sk, sv, std::true_type{}, std::true_type{});
  };

  // 4 waves, hot step m: S^T of tile m (as in slots), then the softmax of
  // tile m interleaved with O^T += V^T P^T of tile m-1 (pin, its P from the
  // previous step), writing P of tile m to pout. The two do not depend on
  // each other, and a wave alone on its SIMD has no partner whose matrix
  // work could cover its vector work, so here one wave does both at once:
  // each product slot (its V^T fragment read RA slots ahead, fenced like
  // slots) carries a share of the softmax -- the score shift and row max
  // beside the first half of the products, the exponentials, row sums and
  // bf16 packing beside the second. The arithmetic and its order are those
  // of softmax_hot (row-sum additions in the same order per accumulator; the
  // max is exact in any order). A rescale of the row references reaches O~
  // only after the last product of tile m-1, as in the sequential step.
  auto hot4 = [&](int m, const bf16* sk, bf16* nk, bf16* nv, const bf16* sv,
                  const bf16x8 (&pin)[NKB * 2], bf16x8 (&pout)[NKB * 2]) FA_INLINE {
    static_assert(NWAVES == 8 || NPV == 16 * NKB, "two scores per product slot");
    constexpr int NPVH = NPV / 2;  // slots in each half
    constexpr int RA = 4;          // V^T fragments read this many slots ahead
    open_step(m, nk, nv);
    slots(sk, sv, std::false_type{}, std::true_type{});
    bf16x8 fr[RA + 1];
#pragma unroll
    for (int k = 0; k < RA; ++k) fr[k] = rd_pv(sv, k);
    auto pv = [&](int k) FA_INLINE {
      if (k + RA < NPV) fr[(k + RA) % (RA + 1)] = rd_pv(sv, k + RA);
      const int mb = k % NMB, kk = k / NMB;
      acc[mb] = mma32(fr[k % (RA + 1)], pin[kk], acc[mb]);
    };
    // First half: shift two scores per slot, t = s * cs - fref, and fold
    // them into one of two max chains.
    float mx[2] = {kNegInf, kNegInf};
#pragma unroll
    for (int k = 0; k < NPVH; ++k) {
      pv(k);
      const float t0 = fmaf(sc[(2 * k) / 16][(2 * k) % 16], cs, -fref);
      const float t1 = fmaf(sc[(2 * k + 1) / 16][(2 * k + 1) % 16], cs, -fref);
      sc[(2 * k) / 16][(2 * k) % 16] = t0;
      sc[(2 * k + 1) / 16][(2 * k + 1) % 16] = t1;
      mx[k & 1] = fmaxf(fmaxf(mx[k & 1], t0), t1);
      __builtin_amdgcn_sched_barrier(0);
    }
    float mt = halves_max(fmaxf(mx[0], mx[1]));
    const bool move = __builtin_amdgcn_ballot_w64(mt > kLazy) != 0;
    float alpha = 1.f;
    if (move) {
      // As in softmax_hot; O~ takes alpha below, after tile m-1's products.
      const float delta = mt > kLazy ? mt : 0.f;
#pragma unroll
      for (int e = 0; e < 16 * NKB; ++e) sc[e / 16][e % 16] -= delta;
      alpha = __builtin_amdgcn_exp2f(-delta);
      lpart *= alpha;
      lcorr *= alpha;
      fref += delta;
      mt -= delta;
    }
    // Second half: two probabilities per slot, their row-sum terms and
    // their bf16 pair of the P^T fragment.
    float rp[4] = {0.f, 0.f, 0.f, 0.f};
    u32x4 pu[NKB * 2];
#pragma unroll
    for (int j = 0; j < NPVH; ++j) {
      pv(NPVH + j);
      const int e0 = 2 * j, r0 = e0 % 16;
      const float x0 = __builtin_amdgcn_exp2f(sc[e0 / 16][e0 % 16]);
      const float x1 = __builtin_amdgcn_exp2f(sc[(e0 + 1) / 16][(e0 + 1) % 16]);
      rp[r0 & 3] += x0;
      rp[(r0 + 1) & 3] += x1;
      pu[(e0 / 16) * 2 + r0 / 8][(r0 % 8) / 2] = pack_bf16x2(x0, x1);
      __builtin_amdgcn_sched_barrier(0);
    }
    lpart += (rp[0] + rp[1]) + (rp[2] + rp[3]);
    const float pm = __builtin_amdgcn_exp2f(mt);
    lcorr += __uint_as_float(pack_bf16x2(pm, 0.f) << 16) - pm;
#pragma unroll
    for (int kk = 0; kk < NKB * 2; ++kk) pout[kk] = as_bf16x8(pu[kk]);
    if (move) {
#pragma unroll
      for (int q = 0; q < NMB; ++q) acc[q] *= alpha;
    }
  };

  // Steps [hot_begin, hot_end) are hot for this wave: tile m exists and is
  // needed by the wave (S^T of tile m), and the softmax tile (m for group A,
  // m-1 for group B) is unmasked. Step 0 and the other steps take the
  // general path. Steps run in pairs starting at an odd step, so every loop
  // keeps a fixed stage assignment; all waves run steps 0 .. ntiles, so
  // they pass the same barriers.
  // The hot softmax needs every row's reference set: the first tile every
  // row of the wave sees (tile 0; with a window's lower edge, tile su_lo) is
  // handled by a general step, which for group B is the step after it.
  const int hot_begin = WIN ? max(1, su_lo + 1 + grp) : 1 + grp;
  const int hot_end = min(min(ntiles, s_last + 1), su_hi + grp);
  if (ntiles > 0) issue(K, ld_koff, 0, sK0);
  wait_global_loads();
  // The first loop takes whole pairs only, so a last single step is left to
  // the final loop. (Each group has loops of its own: one shared generic
  // loop makes the compiler spill.)
  if (grp == 0) {
    step_a(0, sK0, sK1, sV0, sV1);
    int m = 1;
    for (; m < hot_begin && m + 1 <= ntiles; m += 2) {
      step_a(m, sK1, sK0, sV1, sV0);
      step_a(m + 1, sK0, sK1, sV0, sV1);
    }
    for (; m + 1 < hot_end; m += 2) {
      if constexpr (NWAVES == 4) {
        // Step m (odd) reads P of m-1 from pf, writes pf2; step m+1 back.
        hot4(m, sK1, sK0, sV1, sV0, pf, pf2);
        hot4(m + 1, sK0, sK1, sV0, sV1, pf2, pf);
      } else {
        hot_a(m, sK1, sK0, sV1, sV0);
        hot_a(m + 1, sK0, sK1, sV0, sV1);
      }
    }
    for (; m <= ntiles; m += 2) {
      step_a(m, sK1, sK0, sV1, sV0);
      if (m + 1 > ntiles) break;
      step_a(m + 1, sK0, sK1, sV0, sV1);
    }
  } else {
    step_b(0, sK0, sK1, sV0, sV1);
    int m = 1;
    for (; m < hot_begin && m + 1 <= ntiles; m += 2) {
      step_b(m, sK1, sK0, sV1, sV0);
      step_b(m + 1, sK0, sK1, sV0, sV1);
    }
    for (; m + 1 < hot_end; m += 2) {
      hot_b(m, sK1, sK0, sV1, sV0);
      hot_b(m + 1, sK0, sK1, sV0, sV1);
    }
    for (; m <= ntiles; m += 2) {
      step_b(m, sK1, sK0, sV1, sV0);
      if (m + 1 > ntiles) break;
      step_b(m + 1, sK0, sK1, sV0, sV1);
    }
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

template <int D, int BC>
hipError_t launch_d(const Params& p, hipStream_t s) {
  constexpr int NW = D == 256 ? 4 : 8;
  const int t_r = (p.n + 32 * NW - 1) / (32 * NW);
  const long long total = (long long)t_r * p.batch * p.heads;
  dim3 grid((unsigned)total), block(NW * 64);
  return dispatch_mask_win(p, [&](auto causal, auto sparse, auto win) {
    // Block-sparse masks reach only the 4-wave form (d = 256).
    if constexpr (decltype(sparse)::value && NW != 4) {
      return hipErrorInvalidValue;
    } else {
      hipLaunchKernelGGL((fwd_bf16_kernel<D, BC, decltype(causal)::value, decltype(sparse)::value,
                                          decltype(win)::value, NW>),
                         grid, block, 0, s, p);
      return hipGetLastError();
    }
  });
}

}  // namespace

hipError_t launch_fwd_bf16(const Params& p, int d, hipStream_t s) {
  switch (d) {
    case 64: return launch_fwd_bf16_d64(p, d, s);
    // Block-sparse masks take the 4-wave kernel: its 128-row workgroups lie
    // in one block row of the mask.
    case 128: return p.blk != nullptr ? launch_fwd_bf16_d64(p, d, s) : launch_d<128, 64>(p, s);
    // d = 256: 4-wave workgroups of 128 rows, one block row of a block mask.
    case 256: return launch_d<256, 64>(p, s);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace fa
