// Attention backward, dK/dV part, d = 256: key-outer, software-pipelined
// within each wave.
//
// Method as in fa_bwd_bf16.hip: recomputation from the saved row statistic
// (page 1, "注意力为什么受限于显存带宽：用算术强度与分块把 FlashAttention 推导清楚",
// section 八; page 2, "4. FlashAttention 深度剖析", 4.3.4), with
//     dV = P^T dO,  dP = dO V^T,  dS = P * (dP - D),  dK = scale dS^T Q,
// -dP = dO (-V)^T formed on the matrix cores, G = D - dP = D + (-dP) by
// one vector add per element, and P * G = -dS accumulated, so dK comes out
// negated and is scaled by -scale. (Starting the chain from D instead, as
// the d <= 128 kernel does, needs a 16-register copy of D beside the chains,
// and at d = 256 that pushes the K and V fragments out to scratch.)
//
// Layout: a workgroup owns 128 keys (32 per wave) and their dK, dV
// accumulators (256 registers per lane, AGPRs); each wave holds its K and V
// rows as the B operands of S = Q K^T and G (128 VGPRs). The results hold one
// key per lane and 16 queries, the B-operand layout of dV^T += dO^T P and
// dK^T += Q^T (-dS), so P and -dS go to the matrix cores as packed bf16.
// With that much state a SIMD runs one wave, which overlaps its own vector
// and matrix work: step m forms S and G of query tile m, then runs the dV and
// dK products of tile m-1 with P and -dS of tile m computed in the slots
// between them. Query tiles (Q, dO, and their L log2 e and D values) go from
// HBM straight into three LDS stages, row-major with the swizzle that serves
// both the row reads (A operands of S and G) and the transposing reads
// (A operands dO^T and Q^T); tile m is read row-wise in step m and
// transposed in step m+1, while tile m+1 streams into the third stage.
#include <type_traits>

#include "fa_device.h"

namespace fa {

namespace {

constexpr int kThreads = 256;
constexpr int kBKV = 128;  // keys per workgroup (4 waves x 32)
constexpr int kD = 256;
constexpr int kBQ = 32;    // queries per tile

template <bool CAUSAL, bool SPARSE>
__global__ __launch_bounds__(kThreads, 1) void bwd_dkdv_d256_kernel(Params p) {
  constexpr int D = kD;
  constexpr int BQ = kBQ;
  constexpr int CH = D / 8;             // 16-byte chunks per row
  constexpr int ROWB = D * 2;           // bytes per row
  constexpr int TILE = BQ * D;          // elements per Q or dO tile
  constexpr int TILEB = TILE * 2;       // bytes per Q or dO tile
  constexpr int LPW = TILEB / 1024 / 4; // 1 KB wave loads per tensor per wave
  constexpr int RPL = 1024 / ROWB;      // rows per 1 KB load
  constexpr int ND = D / 16;            // reduction steps of S and G
  constexpr int NMB = D / 32;           // 32-row blocks of dK^T and dV^T
  constexpr int HB = 2;                 // block flip of the +8-row half (see toff)
  constexpr int SV = 2 * TILE;          // stage offset (elements) of L and D
  constexpr int STAGE = 2 * TILE + 2 * BQ * 2;  // Q, dO, L (BQ floats), D
  static_assert(LPW * 4 * 1024 == TILEB && RPL == 2 && LPW == 4, "tile split");

  __shared__ __attribute__((aligned(1024))) bf16 sS0[STAGE];
  __shared__ __attribute__((aligned(1024))) bf16 sS1[STAGE];
  __shared__ __attribute__((aligned(1024))) bf16 sS2[STAGE];
  __shared__ int sblk[SPARSE ? kMaxBlocks : 1];

  const int tid = threadIdx.x;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
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

  const int kv_lim = kv_limit(p, b, n);
  const int k0 = kt * kBKV;
  const int mykey = k0 + w * 32 + c;
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
    // K and -V rows of this wave as B fragments: [mykey][kd*16 + h*8 + e].
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
        vf[kd] = as_bf16x8(kok ? (bb ^ 0x80008000u) : z);
      }
    }

    // Out-of-range lanes of a partial tile may leave their LDS bytes as they
    // were, so the stages start as zeros: whatever a masked row holds is then
    // finite, and its zero probability and zero dS contribute exactly 0.
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
      __syncthreads();  // the zeros land before any wave's tile loads
    }

    // The mask, applied on the masked steps: a pair (query q, key) is hidden
    // iff q < qlo or q >= qhi, the queries that see this lane's key (qlo = n
    // for keys at or past the key limit). Query tiles [tb, te) hold every
    // query some key of the workgroup is seen by, tiles [iu0, iu1) only
    // queries that see all of its keys (the bounds are non-decreasing in the
    // key); rows past n are always masked.
    const Band<CAUSAL> band = make_band<CAUSAL>(p, n, kv_lim);
    const int qlo = band.qlo(mykey), qhi = band.qhi(mykey);
    const int k_last = min(k0 + kBKV, kv_lim) - 1;
    const int tb = band.qlo(k0) / BQ;
    const int te = (band.qhi(k_last) + BQ - 1) / BQ;
    const int iu0 = (band.qlo(k0 + kBKV - 1) + BQ - 1) / BQ;
    const int iu1 = band.qhi(k0) / BQ;

    // Per-lane LDS element offsets within a tile (see fa_bwd_dq_bf16.hip):
    // row reads at rbase ^ (kd << 4); transposing reads at tbase ^ (mb << 5),
    // the second read of a fragment (rows +8) in block mb ^ HB.
    const int rbase = c * D + ((h ^ swz_both<D>(c)) << 3);
    int tbase;
    {
      const int trow = h * 4 + ((c & 15) >> 2);
      const int tcol = 16 * (c >> 4) + 4 * (c & 3);
      tbase = trow * D + ((((tcol >> 3) ^ swz_both<D>(trow)) << 3) | (tcol & 7));
    }
    // The bases pass through an empty asm once per use site, so the XORs are
    // redone where they are needed instead of being hoisted into 24
    // registers held across the sweep.
    auto opaque = [&](int x) FA_INLINE {
      asm volatile("" : "+v"(x));
      return x;
    };

    // S = Q K'^T and -dP = dO (-V)^T of the tile in stage st (lane = key,
    // rows 8*(r/4) + 4h + r%4 of the 32 queries), in VGPRs. A fragments are
    // read two products ahead through a ring of three, pinned by the fences.
    auto scores = [&](const bf16* st, f32x16& s, f32x16& g) FA_INLINE {
      const bf16* sq = st;
      const bf16* sg = st + TILE;
      const int rb = opaque(rbase);
      auto roff = [&](int kd) FA_INLINE { return rb ^ (kd << 4); };
      bf16x8 qa[3], ga[3];
      qa[0] = as_bf16x8(ld16(sq + roff(0)));
      ga[0] = as_bf16x8(ld16(sg + roff(0)));
      qa[1] = as_bf16x8(ld16(sq + roff(1)));
      ga[1] = as_bf16x8(ld16(sg + roff(1)));
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int kd = 0; kd < ND; ++kd) {
        if (kd + 2 < ND) {
          qa[(kd + 2) % 3] = as_bf16x8(ld16(sq + roff(kd + 2)));
          ga[(kd + 2) % 3] = as_bf16x8(ld16(sg + roff(kd + 2)));
        }
        if (kd == 0) {
          s = mma32_v0w(qa[0], kf[0]);
          g = mma32_v0w(ga[0], vf[0]);
        } else {
          s = mma32_vw(qa[kd % 3], kf[kd], s);
          g = mma32_vw(ga[kd % 3], vf[kd], g);
        }
        __builtin_amdgcn_sched_barrier(0);
      }
      mfma_drain();
    };

    // Transposed fragment (dO^T or Q^T, tensor at t) for dK/dV block mb and
    // query chunk qc (16 queries), tb an opaque copy of tbase.
    auto rd_t = [&](const bf16* t, int tb, int mb, int qc) FA_INLINE {
      const u32x2 lo = ds_read_tr16(t + qc * 16 * D + (tb ^ (mb << 5)));
      const u32x2 hi = ds_read_tr16(t + (qc * 16 + 8) * D + (tb ^ ((mb ^ HB) << 5)));
      return as_bf16x8(u32x4{lo[0], lo[1], hi[0], hi[1]});
    };
    // Product slot k of a tile whose Q, dO are in stage st: dV^T (k / 8 even)
    // or -dK^T (odd) of block mb = k % 8 and chunk qc = k / 16, so the two
    // products of one accumulator are sixteen slots apart.
    auto frag = [&](const bf16* st, int tb, int k) FA_INLINE {
      const int mb = k % NMB, qc = k / (2 * NMB), isk = (k / NMB) & 1;
      return rd_t(isk ? st : st + TILE, tb, mb, qc);
    };
    auto product = [&](int k, bf16x8 a, const bf16x8 (&pf)[2], const bf16x8 (&sf)[2])
        FA_INLINE {
      const int mb = k % NMB, qc = k / (2 * NMB);
      if ((k / NMB) & 1) dk[mb] = mma32(a, sf[qc], dk[mb]);
      else dv[mb] = mma32(a, pf[qc], dv[mb]);
    };
    // All 32 products of a tile, their transposed fragments read two slots
    // ahead through a ring of three (fenced: hoisting every read would hold
    // 32 fragments at once).
    auto products = [&](const bf16* st, const bf16x8 (&pf)[2], const bf16x8 (&sf)[2])
        FA_INLINE {
      constexpr int NS = 4 * NMB;
      const int tb = opaque(tbase);
      bf16x8 fr[3];
      fr[0] = frag(st, tb, 0);
      fr[1] = frag(st, tb, 1);
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int k = 0; k < NS; ++k) {
        if (k + 2 < NS) fr[(k + 2) % 3] = frag(st, tb, k + 2);
        product(k, fr[k % 3], pf, sf);
        __builtin_amdgcn_sched_barrier(0);
      }
    };

    // P = exp2(S c - L log2 e) and -dS = P (D - dP) of element r, query
    // q0 + 8*(r/4) + 4h + r%4 (lo, hi: this lane's visible queries, relative
    // to q0 + 4h); a hidden pair gets P = 0 and -dS = 0.
    auto pds = [&](const f32x16& s, const f32x16& g, int r, float l, float dv_, int lo, int hi,
                   float& pr, float& x, auto mask_tag) FA_INLINE {
      const int off = (r >> 2) * 8 + (r & 3);
      const float sv = (decltype(mask_tag)::value && (off < lo || off >= hi)) ? kNegInf : s[r];
      pr = __builtin_amdgcn_exp2f(fmaf(sv, cs, -l));
      x = pr * (g[r] + dv_);
    };
    // L log2 e (v = 0) or D (v = 1) of the queries of element group gi.
    auto read_l = [&](const bf16* st, int gi, int v = 0) FA_INLINE {
      return *reinterpret_cast<const f32x4*>(reinterpret_cast<const float*>(st + SV) + v * BQ +
                                             gi * 8 + h * 4);
    };
    // The whole tile's P and -dS as bf16 B fragments: chunk qc holds
    // elements qc*8 .. qc*8+7.
    auto pds_tile = [&](const bf16* st, const f32x16& s, const f32x16& g, int q0,
                        bf16x8 (&pf)[2], bf16x8 (&sf)[2], auto mask_tag) FA_INLINE {
      const int lo = qlo - (q0 + 4 * h), hi = qhi - (q0 + 4 * h);
      u32x4 pu[2], su[2];
#pragma unroll
      for (int gi = 0; gi < 4; ++gi) {
        const f32x4 l4 = read_l(st, gi);
        const f32x4 d4 = read_l(st, gi, 1);
#pragma unroll
        for (int i = 0; i < 4; i += 2) {
          float p0, x0, p1, x1;
          pds(s, g, gi * 4 + i, l4[i], d4[i], lo, hi, p0, x0, mask_tag);
          pds(s, g, gi * 4 + i + 1, l4[i + 1], d4[i + 1], lo, hi, p1, x1, mask_tag);
          pu[gi >> 1][((gi & 1) * 4 + i) >> 1] = pack_bf16x2(p0, p1);
          su[gi >> 1][((gi & 1) * 4 + i) >> 1] = pack_bf16x2(x0, x1);
        }
      }
      pf[0] = as_bf16x8(pu[0]);
      pf[1] = as_bf16x8(pu[1]);
      sf[0] = as_bf16x8(su[0]);
      sf[1] = as_bf16x8(su[1]);
    };

    // Hot phase two: the products of the previous tile (stage prev, fragments
    // pfp, sfp) with P and -dS of this unmasked tile (stage cur) in their
    // slots, two slots per element pair (transposed fragments read two slots
    // ahead; the packed pairs are pinned to their slots, or the compiler
    // sinks the arithmetic into the next step, whose products read it).
    auto products_with_pds = [&](const bf16* prev, const bf16x8 (&pfp)[2],
                                 const bf16x8 (&sfp)[2], const bf16* cur, const f32x16& s,
                                 const f32x16& g, bf16x8 (&pfn)[2], bf16x8 (&sfn)[2])
        FA_INLINE {
      constexpr int NS = 4 * NMB;  // 32 slots, 16 elements
      const int tb = opaque(tbase);
      bf16x8 fr[3];
      fr[0] = frag(prev, tb, 0);
      fr[1] = frag(prev, tb, 1);
      f32x4 l4 = read_l(cur, 0), d4 = read_l(cur, 0, 1);
      u32x4 pu[2], su[2];
      float p0 = 0.f, x0 = 0.f;
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int k = 0; k < NS; ++k) {
        if (k + 2 < NS) fr[(k + 2) % 3] = frag(prev, tb, k + 2);
        product(k, fr[k % 3], pfp, sfp);
        const int r = k / 2, gi = r / 4, i = r % 4;
        if ((k & 1) == 0) {
          if (i == 0 && gi > 0) {
            l4 = read_l(cur, gi);
            d4 = read_l(cur, gi, 1);
          }
          float pr, x;
          pds(s, g, r, l4[i], d4[i], 0, 0, pr, x, std::false_type{});
          if ((r & 1) == 0) {
            p0 = pr;
            x0 = x;
          } else {
            const int j = (gi & 1) * 2 + (i >> 1);
            pu[gi >> 1][j] = pack_bf16x2(p0, pr);
            su[gi >> 1][j] = pack_bf16x2(x0, x);
            asm volatile("" : "+v"(pu[gi >> 1][j]), "+v"(su[gi >> 1][j]));
          }
        }
        __builtin_amdgcn_sched_barrier(0);
      }
      pfn[0] = as_bf16x8(pu[0]);
      pfn[1] = as_bf16x8(pu[1]);
      sfn[0] = as_bf16x8(su[0]);
      sfn[1] = as_bf16x8(su[1]);
    };

    auto sweep = [&](const auto& tiles) FA_INLINE {
      const int ns = tiles.count;
      if (ns == 0) return;
      // Steps [su0, su1) hold only queries that see every key of the
      // workgroup.
      int su0, su1;
      tiles.steps_of(iu0, iu1, su0, su1);
      for (int gq = 0; gq < p.group; ++gq) {
        // Query head gq of the group: its Q, dO and row vectors (work entry
        // of query head hk * group + gq).
        const int bh = b * p.heads + hk * p.group + gq;
        const size_t base = span_row0(p, sp, p.heads, hk * p.group + gq) * D;
        const auto rq = buffer_rsrc(static_cast<const bf16*>(p.q) + base, n * ROWB);
        const auto rg = buffer_rsrc(static_cast<const bf16*>(p.d_o) + base, n * ROWB);
        const auto rl = buffer_rsrc(p.l2vec + (size_t)bh * p.n_pad, p.n_pad * 4);
        const auto rd = buffer_rsrc(p.dvec + (size_t)bh * p.n_pad, p.n_pad * 4);
        // Waves may still be reading the previous head's last tile from the
        // stages; every wave is past it before they are refilled.
        if (gq > 0) __syncthreads();
        // Loads of query tile it into stage st: wave w fills rows
        // [w*LPW*RPL, (w+1)*LPW*RPL) of the Q and dO tiles (lane l of a 1 KB
        // load writes physical chunk l % CH of row l / CH, holding logical
        // chunk (l % CH) ^ swz_both(row); load i covers rows 2i past load
        // 0's, whose swizzle differs by a constant XOR of the chunk index).
        // The descriptors span the head's n rows, so rows past n are never
        // read. Wave 0 also loads the tile's L log2 e and D values (the
        // vectors are padded per head, so a tile is always in range).
        auto issue = [&](int it, bf16* st) FA_INLINE {
          int lid;
          asm volatile("v_mbcnt_lo_u32_b32 %0, -1, 0\n\tv_mbcnt_hi_u32_b32 %0, -1, %0"
                       : "=v"(lid));
          const int row = w * LPW * RPL + lid / CH;
          const int ob = (row * D + ((lid % CH) ^ swz_both<D>(row)) * 8) * 2;
          const int qb0 = it * BQ * ROWB;
#pragma unroll
          for (int i = 0; i < LPW; ++i) {
            const int o = qb0 + (ob ^ (((10 * (i & 1) + 4 * (i >> 1)) << 4) | (i << 10)));
            bload_lds16(rq, o, st + (w * LPW + i) * RPL * D);
            bload_lds16(rg, o, st + TILE + (w * LPW + i) * RPL * D);
          }
          if (w == 0 && lane < BQ / 4) {
            bload_lds16(rl, it * BQ * 4 + lane * 16, st + SV);
            bload_lds16_at(rd, it * BQ * 4 + lane * 16, st + SV, BQ * 4);
          }
        };
        // Step m on query tile tiles.tile(m): stage cur holds it, prev tile
        // m-1 and nxt receives tile m+1 (it held tile m-2, last read in step
        // m-1). Each wave waits for its own loads of tile m, then the barrier
        // makes every wave's loads visible. Every step runs the dV, dK
        // products of the previous tile (fragments pfp, sfp): zeros before
        // the first, which add exactly 0 (the stage holds finite data).
        // A step T-1 = ns past the last tile only finishes tile ns-1; the
        // scores it forms from its stage's stale data are dropped. (Branches
        // around the products, or a separate finishing body, put the
        // accumulators through control-flow merges, and with all 256 AGPRs
        // taken by them every copy there went to scratch.)
        bf16x8 pfp[2], sfp[2];
#pragma unroll
        for (int j = 0; j < 2; ++j) {
          pfp[j] = as_bf16x8(u32x4{0u, 0u, 0u, 0u});
          sfp[j] = as_bf16x8(u32x4{0u, 0u, 0u, 0u});
        }
        auto open = [&](int m, bf16* nxt) FA_INLINE {
          wait_global_loads();
          __syncthreads();
          if (m + 1 < ns) issue(tiles.tile(m + 1), nxt);
        };
        auto gstep = [&](int m, bf16* cur, bf16* prev, bf16* nxt) FA_INLINE {
          open(m, nxt);
          const bool tail = m == ns;
          const int q0 = tail ? 0 : tiles.tile(m) * BQ;
          const bool full = tail || (m >= su0 && m < su1);
          f32x16 s, g;
          scores(cur, s, g);
          products(prev, pfp, sfp);
          if (full) pds_tile(cur, s, g, q0, pfp, sfp, std::false_type{});
          else pds_tile(cur, s, g, q0, pfp, sfp, std::true_type{});
        };
        auto hstep = [&](int m, bf16* cur, bf16* prev, bf16* nxt) FA_INLINE {
          open(m, nxt);
          f32x16 s, g;
          scores(cur, s, g);
          bf16x8 pfn[2], sfn[2];
          products_with_pds(prev, pfp, sfp, cur, s, g, pfn, sfn);
          pfp[0] = pfn[0];
          pfp[1] = pfn[1];
          sfp[0] = sfn[0];
          sfp[1] = sfn[1];
        };
        // Steps run in groups of three from a multiple of three (each stage
        // assignment has its own code): general steps up to the first
        // multiple of three past su0, hot groups while they lie below su1,
        // general steps to the end (T = ns + 1 steps in all).
        const int T = ns + 1;
        const int hb = min(T, (su0 + 3) / 3 * 3);
        issue(tiles.tile(0), sS0);
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
        // m is a multiple of three here unless the first loop stopped at T.
        for (; m < T; m += 3) {
          gstep(m, sS0, sS2, sS1);
          if (m + 1 >= T) break;
          gstep(m + 1, sS1, sS0, sS2);
          if (m + 2 >= T) break;
          gstep(m + 2, sS2, sS1, sS0);
        }
      }  // query heads of the group
    };
    // Query tiles from the last down: in a causal sweep every workgroup of
    // a head then starts at the same tile, so the workgroups running side by
    // side read the same Q and dO tiles at about the same time (from the
    // diagonal up they start 128 rows apart, and 32 of them on one L2 keep
    // about 4 MB of d = 256 tiles in flight).
    if constexpr (SPARSE) {
      // The workgroup's 128 keys are one block column of the mask.
      const int nl = stage_blocks(col_blocks(p, k0 / kBlock), sblk, tid, kThreads, p.nb);
      sweep(reversed(sparse_tiles<kBlock / BQ>(sblk, nl, tb, te)));
    } else {
      sweep(reversed(dense_tiles(tb, te)));
    }
  }

  // dK = scale * (dS^T Q), dV as accumulated.
  if (mykey < n) {
    const float ks = -p.scale;  // dk holds -dS^T Q
#pragma unroll
    for (int mb = 0; mb < NMB; ++mb)
#pragma unroll
      for (int gi = 0; gi < 4; ++gi) {
        const size_t off = (size_t)mykey * D + mb * 32 + gi * 8 + h * 4;
        u32x2 uk, uv;
        uk[0] = pack_bf16x2(dk[mb][gi * 4 + 0] * ks, dk[mb][gi * 4 + 1] * ks);
        uk[1] = pack_bf16x2(dk[mb][gi * 4 + 2] * ks, dk[mb][gi * 4 + 3] * ks);
        uv[0] = pack_bf16x2(dv[mb][gi * 4 + 0], dv[mb][gi * 4 + 1]);
        uv[1] = pack_bf16x2(dv[mb][gi * 4 + 2], dv[mb][gi * 4 + 3]);
        *reinterpret_cast<u32x2*>(dK + off) = uk;
        *reinterpret_cast<u32x2*>(dV + off) = uv;
      }
  }
}

}  // namespace

hipError_t launch_bwd_dkdv_bf16_d256(const Params& p, int d, hipStream_t s) {
  if (d != kD) return hipErrorInvalidValue;
  const int t_c = (p.n + kBKV - 1) / kBKV;
  const long long total = (long long)t_c * p.batch * p.heads_kv;
  dim3 grid((unsigned)total), block(kThreads);
  return dispatch_mask(p, [&](auto causal, auto sparse) {
    hipLaunchKernelGGL((bwd_dkdv_d256_kernel<decltype(causal)::value, decltype(sparse)::value>),
                       grid, block, 0, s, p);
    return hipGetLastError();
  });
}

}  // namespace fa
