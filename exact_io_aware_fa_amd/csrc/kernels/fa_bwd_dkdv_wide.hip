// Attention backward, dK/dV part, d = 128 with 64 keys per wave.
//
// Method as in fa_bwd_bf16.hip: recomputation from the saved row statistic
// (page 1, "注意力为什么受限于显存带宽：用算术强度与分块把 FlashAttention 推导清楚",
// section 八; page 2, "4. FlashAttention 深度剖析", 4.3.4), with
//     dV = P^T dO,  dP = dO V^T,  dS = P * (dP - D),  dK = scale dS^T Q,
// -dP = dO (-V)^T formed on the matrix cores, G = D - dP by one vector add
// per element, and P * G = -dS accumulated (dK comes out negated and is
// scaled by -scale).
//
// Why 64 keys: every product here reads its A operand from LDS (a 1 KB
// fragment of Q, dO, Q^T or dO^T) and its B operand from registers (K and V
// rows, P and -dS). With 32 keys per wave that is one fragment per product,
// and LDS operand reads bound the 32-key kernel. A wave that owns two blocks
// of 32 keys uses each fragment for two products, halving the LDS traffic
// per product. The price is registers: K and V fragments (128 VGPRs) and
// dK, dV accumulators (256 AGPRs) for 64 keys leave room for one S/G
// register set and the packed P, -dS of half a tile. So the pipeline runs
// by half tiles: step m forms the scores of tile m, then the products of
// the second 16 queries of tile m-1 with P and -dS of the first 16 queries
// of tile m computed in their slots, then the products of those first 16
// queries with P and -dS of the second 16 computed in theirs.
//
// A workgroup is 4 waves (one per SIMD) and owns 256 keys; query tiles of
// 32 rows (Q, dO, L log2 e, D) go from HBM straight into three LDS stages
// (tile m read in step m and transposed in steps m and m+1, tile m+1
// streaming in), row-major with the swizzle that serves both the row reads
// and the transposing reads, one barrier per step. Block-sparse calls keep
// the 128-key kernel: 256 keys span two block columns of the mask, whose
// query-block lists would have to be merged. So do windowed calls: at each
// edge of the window a 256-key workgroup has twice the partly visible query
// tiles of a 128-key one, and measured slower.
#include <type_traits>

#include "fa_device.h"

namespace fa {

namespace {

constexpr int kThreads = 256;
constexpr int kBKV = 256;  // keys per workgroup (4 waves x 64)
constexpr int kD = 128;
constexpr int kBQ = 32;    // queries per tile

template <bool CAUSAL>
__global__ __launch_bounds__(kThreads, 1) void bwd_dkdv_wide_kernel(Params p) {
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
  constexpr int HB = 2;                 // block flip of the +8-row half (see tbase)
  constexpr int NKB = 2;                // key blocks of 32 per wave
  constexpr int SV = 2 * TILE;          // stage offset (elements) of L and D
  constexpr int STAGE = 2 * TILE + 2 * BQ * 2;  // Q, dO, L (BQ floats), D
  static_assert(LPW == 2 && RPL == 4, "tile split");

  __shared__ __attribute__((aligned(1024))) bf16 sS0[STAGE];
  __shared__ __attribute__((aligned(1024))) bf16 sS1[STAGE];
  __shared__ __attribute__((aligned(1024))) bf16 sS2[STAGE];

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
  const int kw0 = k0 + w * 64;  // this wave's keys: kw0 + kb * 32 + c
  const float cs = p.c;
  // A negative scale is applied by negating K (exact in bf16): the scores
  // use K' = -K with |scale|, and dK = scale dS^T Q with the true Q.
  const uint32_t kflip = p.q_neg ? 0x80008000u : 0u;

  f32x16 dk[NKB][NMB], dv[NKB][NMB];
#pragma unroll
  for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
    for (int mb = 0; mb < NMB; ++mb) {
      dk[kb][mb] = f32x16{};
      dv[kb][mb] = f32x16{};
    }

  if (k0 < kv_lim) {
    // K and -V rows of this wave as B fragments: [key][kd*16 + h*8 + e].
    // Rows past the key limit are read clamped and replaced by zeros.
    bf16x8 kf[NKB][ND], vf[NKB][ND];
#pragma unroll
    for (int kb = 0; kb < NKB; ++kb) {
      const int key = kw0 + kb * 32 + c;
      const bool kok = key < kv_lim;
      const int kr = kok ? key : kv_lim - 1;
#pragma unroll
      for (int kd = 0; kd < ND; ++kd) {
        const u32x4 z = {0u, 0u, 0u, 0u};
        const u32x4 a = ld16(K + (size_t)kr * D + kd * 16 + h * 8);
        const u32x4 bb = ld16(V + (size_t)kr * D + kd * 16 + h * 8);
        kf[kb][kd] = as_bf16x8(kok ? (a ^ kflip) : z);
        vf[kb][kd] = as_bf16x8(kok ? (bb ^ 0x80008000u) : z);
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
    // iff q < qlo or q >= qhi, the queries that see the lane's key of block
    // kb (qlo = n for keys at or past the key limit). Query tiles [tb, te)
    // hold every query some key of the workgroup is seen by, tiles
    // [iu0, iu1) only queries that see all of its keys (the bounds are
    // non-decreasing in the key); rows past n are always masked.
    const Band<CAUSAL> band = make_band<CAUSAL>(p, n, kv_lim);
    int qlo[NKB], qhi[NKB];
#pragma unroll
    for (int kb = 0; kb < NKB; ++kb) {
      qlo[kb] = band.qlo(kw0 + kb * 32 + c);
      qhi[kb] = band.qhi(kw0 + kb * 32 + c);
    }
    const int k_last = min(k0 + kBKV, kv_lim) - 1;
    const int tb = band.qlo(k0) / BQ;
    const int te = (band.qhi(k_last) + BQ - 1) / BQ;
    const int iu0 = (band.qlo(k0 + kBKV - 1) + BQ - 1) / BQ;
    const int iu1 = band.qhi(k0) / BQ;

    // Per-lane LDS element offsets within a tile (see fa_bwd_dq_bf16.hip):
    // row reads at rbase ^ (kd << 4); transposing reads at tbase ^ (mb << 5),
    // the second read of a fragment (rows +8) in block mb ^ HB. The bases
    // pass through an empty asm at each use site, so the XORs are redone
    // there instead of being hoisted into registers held across the sweep.
    const int rbase = c * D + ((h ^ swz_both<D>(c)) << 3);
    int tbase;
    {
      const int trow = h * 4 + ((c & 15) >> 2);
      const int tcol = 16 * (c >> 4) + 4 * (c & 3);
      tbase = trow * D + ((((tcol >> 3) ^ swz_both<D>(trow)) << 3) | (tcol & 7));
    }
    auto opaque = [&](int x) FA_INLINE {
      asm volatile("" : "+v"(x));
      return x;
    };

    // S = Q K'^T and -dP = dO (-V)^T of the tile in stage st for both key
    // blocks (lane = key, rows 8*(r/4) + 4h + r%4 of the 32 queries), in
    // VGPRs: each Q and dO fragment (read two steps ahead through a ring of
    // three, fenced) feeds two products.
    auto scores = [&](const bf16* st, f32x16 (&s)[NKB], f32x16 (&g)[NKB]) FA_INLINE {
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
#pragma unroll
        for (int kb = 0; kb < NKB; ++kb) {
          if (kd == 0) {
            s[kb] = mma32_v0w(qa[0], kf[kb][0]);
            g[kb] = mma32_v0w(ga[0], vf[kb][0]);
          } else {
            s[kb] = mma32_vw(qa[kd % 3], kf[kb][kd], s[kb]);
            g[kb] = mma32_vw(ga[kd % 3], vf[kb][kd], g[kb]);
          }
        }
        __builtin_amdgcn_sched_barrier(0);
      }
      mfma_drain();
    };

    // Transposed fragment (dO^T or Q^T, tensor at t) for dK/dV block mb and
    // query chunk qc (16 queries); tb is an opaque copy of tbase.
    auto rd_t = [&](const bf16* t, int tb, int mb, int qc) FA_INLINE {
      const u32x2 lo = ds_read_tr16(t + qc * 16 * D + (tb ^ (mb << 5)));
      const u32x2 hi = ds_read_tr16(t + (qc * 16 + 8) * D + (tb ^ ((mb ^ HB) << 5)));
      return as_bf16x8(u32x4{lo[0], lo[1], hi[0], hi[1]});
    };

    // L log2 e (v = 0) or D (v = 1) of the queries of element group gi.
    auto read_l = [&](const bf16* st, int gi, int v) FA_INLINE {
      return *reinterpret_cast<const f32x4*>(reinterpret_cast<const float*>(st + SV) + v * BQ +
                                             gi * 8 + h * 4);
    };
    // P = exp2(S c - L log2 e) and -dS = P (D - dP) of element r of key
    // block kb (query q0 + 8*(r/4) + 4h + r%4); a hidden pair gets 0 and 0.
    auto pds = [&](const f32x16& s, const f32x16& g, int r, float l, float d_, int lo, int hi,
                   float& pr, float& x, auto mask_tag) FA_INLINE {
      const int off = (r >> 2) * 8 + (r & 3);
      const float sv = (decltype(mask_tag)::value && (off < lo || off >= hi)) ? kNegInf : s[r];
      pr = __builtin_amdgcn_exp2f(fmaf(sv, cs, -l));
      x = pr * (g[r] + d_);
    };

    // Chunk products: for query chunk qc (16 queries) of the tile whose Q, dO
    // are in stage st, the 16 dV and dK products (slot k: block mb = k / 4;
    // dV of key block 0, 1, then dK of key block 0, 1), fragments pf, sf.
    // The dO^T and Q^T fragments of block mb+1 are read one block ahead.
    // Each slot k also runs slot(k), vector work placed there (fenced).
    auto chunk = [&](const bf16* st, int tb, int qc, const bf16x8 (&pf)[NKB],
                     const bf16x8 (&sf)[NKB], auto&& slot) FA_INLINE {
      const bf16* so = st + TILE;
      bf16x8 fo[2], fq[2];
      fo[0] = rd_t(so, tb, 0, qc);
      fq[0] = rd_t(st, tb, 0, qc);
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int k = 0; k < 4 * NMB; ++k) {
        const int mb = k / 4, j = k % 4;
        if (j == 0 && mb + 1 < NMB) {
          fo[(mb + 1) % 2] = rd_t(so, tb, mb + 1, qc);
          fq[(mb + 1) % 2] = rd_t(st, tb, mb + 1, qc);
        }
        if (j < 2) dv[j][mb] = mma32(fo[mb % 2], pf[j], dv[j][mb]);
        else dk[j - 2][mb] = mma32(fq[mb % 2], sf[j - 2], dk[j - 2][mb]);
        slot(k);
        __builtin_amdgcn_sched_barrier(0);
      }
    };
    // P and -dS of query chunk qc of a tile (scores s, g; L, D in stage st),
    // one element per slot k (element qc*8 + k % 8 of key block k / 8), packed
    // into pf, sf (bf16 pairs pinned to their slots: the compiler would
    // otherwise move the arithmetic to where the fragments are read).
    struct Pack {
      u32x4 pu[NKB], su[NKB];
      float p0, x0;
      f32x4 l4, d4;
    };
    auto pds_slot = [&](Pack& pk, const bf16* st, const f32x16 (&s)[NKB],
                        const f32x16 (&g)[NKB], int qc, int k, const int (&lo)[NKB],
                        const int (&hi)[NKB], auto mask_tag) FA_INLINE {
      const int kb = k / 8, r = qc * 8 + k % 8, i = r % 4;
      if (k % 4 == 0) {
        pk.l4 = read_l(st, r / 4, 0);
        pk.d4 = read_l(st, r / 4, 1);
      }
      float pr, x;
      pds(s[kb], g[kb], r, pk.l4[i], pk.d4[i], lo[kb], hi[kb], pr, x, mask_tag);
      if ((r & 1) == 0) {
        pk.p0 = pr;
        pk.x0 = x;
      } else {
        const int t = (r % 8) >> 1;
        pk.pu[kb][t] = pack_bf16x2(pk.p0, pr);
        pk.su[kb][t] = pack_bf16x2(pk.x0, x);
        asm volatile("" : "+v"(pk.pu[kb][t]), "+v"(pk.su[kb][t]));
      }
    };

    // Step m on the tile in stage cur (query row q0; `full` masks off): its
    // scores; then the chunk-1 products of the previous tile (stage prev,
    // fragments pf1, sf1, zeros before the first tile) with this tile's
    // chunk-0 P and -dS in their slots; then this tile's chunk-0 products
    // with its chunk-1 P and -dS in their slots, which the next step's
    // products take. A step past the last tile (tail) finishes the last
    // tile's chunk 1; its own P and -dS are fully masked, so its chunk-0
    // products add exactly 0.
    bf16x8 pf1[NKB], sf1[NKB];
    auto run = [&](const bf16* cur, const bf16* prev, int q0, bool tail, auto mask_tag)
        FA_INLINE {
      f32x16 s[NKB], g[NKB];
      scores(cur, s, g);
      int lo[NKB], hi[NKB];
#pragma unroll
      for (int kb = 0; kb < NKB; ++kb) {
        lo[kb] = tail ? 0 : qlo[kb] - (q0 + 4 * h);
        hi[kb] = tail ? 0 : qhi[kb] - (q0 + 4 * h);
      }
      const int tb = opaque(tbase);
      Pack pk0;
      pk0.p0 = pk0.x0 = 0.f;
      chunk(prev, tb, 1, pf1, sf1, [&](int k) FA_INLINE {
        pds_slot(pk0, cur, s, g, 0, k, lo, hi, mask_tag);
      });
      bf16x8 pf0[NKB], sf0[NKB];
#pragma unroll
      for (int kb = 0; kb < NKB; ++kb) {
        pf0[kb] = as_bf16x8(pk0.pu[kb]);
        sf0[kb] = as_bf16x8(pk0.su[kb]);
      }
      Pack pk1;
      pk1.p0 = pk1.x0 = 0.f;
      chunk(cur, tb, 0, pf0, sf0, [&](int k) FA_INLINE {
        pds_slot(pk1, cur, s, g, 1, k, lo, hi, mask_tag);
      });
#pragma unroll
      for (int kb = 0; kb < NKB; ++kb) {
        pf1[kb] = as_bf16x8(pk1.pu[kb]);
        sf1[kb] = as_bf16x8(pk1.su[kb]);
      }
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
        // Waves may still be reading the previous head's last tiles from the
        // stages; every wave is past them before they are refilled.
        if (gq > 0) __syncthreads();
        // Loads of query tile it into stage st: wave w fills rows
        // [w*LPW*RPL, (w+1)*LPW*RPL) of the Q and dO tiles (lane l of a 1 KB
        // load writes physical chunk l % CH of row l / CH, holding logical
        // chunk (l % CH) ^ swz_both(row); load 1 covers rows 4 past load 0's,
        // whose swizzle differs by XOR 4 of the chunk index, and its row
        // step sets bit 10, which load 0's offset leaves clear). The
        // descriptors span the head's n rows, so rows past n are never read.
        // Wave 0 also loads the tile's L log2 e and D values (the vectors are
        // padded per head, so a tile is always in range).
        auto issue = [&](int it, bf16* st) FA_INLINE {
          int lid;
          asm volatile("v_mbcnt_lo_u32_b32 %0, -1, 0\n\tv_mbcnt_hi_u32_b32 %0, -1, %0"
                       : "=v"(lid));
          const int row = w * LPW * RPL + lid / CH;
          const int ob = (row * D + ((lid % CH) ^ swz_both<D>(row)) * 8) * 2;
          const int qb0 = it * BQ * ROWB;
#pragma unroll
          for (int i = 0; i < LPW; ++i) {
            const int o = qb0 + (ob ^ (((4 * i) << 4) | (i << 10)));
            bload_lds16(rq, o, st + (w * LPW + i) * RPL * D);
            bload_lds16(rg, o, st + TILE + (w * LPW + i) * RPL * D);
          }
          if (w == 0 && lane < BQ / 4) {
            bload_lds16(rl, it * BQ * 4 + lane * 16, st + SV);
            bload_lds16_at(rd, it * BQ * 4 + lane * 16, st + SV, BQ * 4);
          }
        };
#pragma unroll
        for (int kb = 0; kb < NKB; ++kb) {
          pf1[kb] = as_bf16x8(u32x4{0u, 0u, 0u, 0u});
          sf1[kb] = as_bf16x8(u32x4{0u, 0u, 0u, 0u});
        }
        // Step m: stage cur holds tile m, prev tile m-1, and tile m+1 goes
        // to nxt, which held tile m-2 (last read in step m-1, before this
        // step's barrier). Each wave waits for its own loads of tile m, then
        // the barrier makes every wave's loads visible. Step ns is the tail.
        // (Loading two tiles ahead through a fourth stage does not work with
        // this compiler: it cannot keep that many LDS-DMA targets apart and
        // waits for every load before some steps' first LDS read.)
        auto step = [&](int m, bf16* cur, bf16* prev, bf16* nxt, auto mask_tag) FA_INLINE {
          wait_global_loads();
          __syncthreads();
          if (m + 1 < ns) issue(tiles.tile(m + 1), nxt);
          const bool tail = m == ns;
          run(cur, prev, tail ? 0 : tiles.tile(m) * BQ, tail, mask_tag);
        };
        // Groups of three steps from a multiple of three (each stage
        // assignment has its own code): masked steps up to the first
        // multiple of three past su0, unmasked groups while they lie below
        // su1, masked steps to the end (T = ns + 1 steps with the tail).
        const int T = ns + 1;
        const int hb = min(T, (su0 + 2) / 3 * 3);
        issue(tiles.tile(0), sS0);
        int m = 0;
        for (; m < hb; m += 3) {
          step(m, sS0, sS2, sS1, std::true_type{});
          if (m + 1 >= hb) { m += 1; break; }
          step(m + 1, sS1, sS0, sS2, std::true_type{});
          if (m + 2 >= hb) { m += 2; break; }
          step(m + 2, sS2, sS1, sS0, std::true_type{});
        }
        if (m == hb && hb % 3 == 0) {
          for (; m + 3 <= su1; m += 3) {
            step(m, sS0, sS2, sS1, std::false_type{});
            step(m + 1, sS1, sS0, sS2, std::false_type{});
            step(m + 2, sS2, sS1, sS0, std::false_type{});
          }
        }
        // m is a multiple of three here unless the first loop stopped at T.
        for (; m < T; m += 3) {
          step(m, sS0, sS2, sS1, std::true_type{});
          if (m + 1 >= T) break;
          step(m + 1, sS1, sS0, sS2, std::true_type{});
          if (m + 2 >= T) break;
          step(m + 2, sS2, sS1, sS0, std::true_type{});
        }
      }  // query heads of the group
    };
    // Query tiles from the last down. In a causal sweep every workgroup of a
    // head then starts at the same (last) tile and ends at its own diagonal,
    // so the workgroups running side by side read the same Q and dO tiles at
    // about the same time and the L2 serves all but the first. (From the
    // diagonal up, neighbouring workgroups start 256 rows apart, and 32 of
    // them on one L2 keep about 4 MB of tiles in flight.)
    sweep(reversed(dense_tiles(tb, te)));
  }

  // dK = scale * (dS^T Q), dV as accumulated.
#pragma unroll
  for (int kb = 0; kb < NKB; ++kb) {
    const int key = kw0 + kb * 32 + c;
    if (key < n) {
      const float ks = -p.scale;  // dk holds -dS^T Q
#pragma unroll
      for (int mb = 0; mb < NMB; ++mb)
#pragma unroll
        for (int gi = 0; gi < 4; ++gi) {
          const size_t off = (size_t)key * D + mb * 32 + gi * 8 + h * 4;
          u32x2 uk, uv;
          uk[0] = pack_bf16x2(dk[kb][mb][gi * 4 + 0] * ks, dk[kb][mb][gi * 4 + 1] * ks);
          uk[1] = pack_bf16x2(dk[kb][mb][gi * 4 + 2] * ks, dk[kb][mb][gi * 4 + 3] * ks);
          uv[0] = pack_bf16x2(dv[kb][mb][gi * 4 + 0], dv[kb][mb][gi * 4 + 1]);
          uv[1] = pack_bf16x2(dv[kb][mb][gi * 4 + 2], dv[kb][mb][gi * 4 + 3]);
          *reinterpret_cast<u32x2*>(dK + off) = uk;
          *reinterpret_cast<u32x2*>(dV + off) = uv;
        }
    }
  }
}

}  // namespace

hipError_t launch_bwd_dkdv_bf16_wide(const Params& p, int d, hipStream_t s) {
  if (d != kD || p.blk != nullptr || p.win_left >= 0 || p.win_right >= 0)
    return hipErrorInvalidValue;
  const int t_c = (p.n + kBKV - 1) / kBKV;
  const long long total = (long long)t_c * p.batch * p.heads_kv;
  dim3 grid((unsigned)total), block(kThreads);
  if (p.causal)
    hipLaunchKernelGGL((bwd_dkdv_wide_kernel<true>), grid, block, 0, s, p);
  else
    hipLaunchKernelGGL((bwd_dkdv_wide_kernel<false>), grid, block, 0, s, p);
  return hipGetLastError();
}

}  // namespace fa
