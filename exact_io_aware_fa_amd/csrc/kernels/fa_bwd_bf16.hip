// Attention backward, dK/dV part: bf16 in/out, fp32 accumulate, for gfx950
// (d = 64 and 128; d = 64 with at most 1024 rows uses fa_bwd_dkdv_d64.hip,
// d = 256 fa_bwd_dkdv_d256.hip).
//
// Method: recomputation from the saved row statistic (page 1, "注意力为什么
// 受限于显存带宽：用算术强度与分块把 FlashAttention 推导清楚", section 八; page 2,
// "4. FlashAttention 深度剖析", 4.3.4): P_ij = exp(scale q_i.k_j - L_i) is
// rebuilt tile by tile and never stored. The gradient formulas are the
// ordinary calculus of softmax attention (the pages name dS, dQ, dK, dV but
// print no formula):
//     dV = P^T dO,  dP = dO V^T,  dS = P * (dP - D),  D_i = <dO_i, O_i>,
//     dK = scale dS^T Q.
// The kernel forms G = D - dP on the matrix cores (dO (-V)^T accumulated
// onto D) and accumulates P * G = -dS, so dK comes out negated and is
// scaled by -scale at the end: the subtraction costs no vector instruction.
// dQ = scale dS K is computed by the query-outer kernel in
// fa_bwd_dq_bf16.hip.
//
// Mapping onto CDNA4:
// * A workgroup is 4 wave64s and owns BKV = 128 keys (32 per wave) and their
//   dK, dV accumulators (fp32) for the whole query sweep; it loops over
//   query tiles of BQ rows (key/value-outer order: dK and dV are each
//   written once, no atomics).
// * Each wave keeps its 32 K and V rows in VGPRs as the B operands of
//   S = Q K^T and dP = dO V^T; the results hold one key per lane and 16
//   queries per 32-query block, which is exactly the B-operand layout of
//   dV^T += dO^T P and dK^T += Q^T dS, so P and dS go to the matrix cores
//   without leaving registers.
// * Query tiles (Q, dO, and their L log2 e and D values) go from HBM
//   straight into LDS through buffer descriptors, row-major with one XOR
//   swizzle that makes both the row reads (A operands of S and dP) and the
//   transposing reads (A operands of dV^T and dK^T, ds_read_b64_tr_b16)
//   conflict-free. Four stages: tile i+2 streams in while tile i+1 is read
//   row-wise and tile i transposed; one barrier per tile.
// * Software pipeline: iteration i computes S and dP of tile i+1 on the
//   matrix cores while the vector units turn S and dP of tile i into P and
//   dS, then accumulates dV and dK of tile i. With one wave per SIMD (the
//   accumulators and K/V fragments need more than half the register file)
//   the overlap has to come from within the wave.
// * The S and dP products write ordinary VGPRs (mma32_v, in fa_device.h), and the
//   results of consecutive tiles alternate between two register sets (the
//   loop is unrolled by four, the period of both the stages and the sets):
//   the vector units read them where they land, with no copy out of the
//   accumulation registers that the dK, dV products use.
#include <type_traits>

#include "fa_device.h"

namespace fa {

namespace {

constexpr int kThreads = 256;
constexpr int kBKV = 128;  // keys per workgroup (4 waves x 32)

// S and dP accumulate in VGPRs (mma32_v, mma32_v0, mma32_vc in fa_device.h):
// this kernel may use more than 256 registers per lane, so the compiler
// gives every matrix builtin the AGPR form, after which the vector units
// could read S and dP only through one v_accvgpr_read per value. The
// assembly products are safe here because every result is first read, and
// its registers first reused, by code of the next pipeline step (hundreds
// of instructions and 16 products later, beyond any required wait states;
// the step keeps its results and accumulator inputs live to its end, see
// body), and each accumulation chain alternates with another, so two
// products of one chain are never adjacent.

template <int D, int NQB, bool CAUSAL, bool SPARSE>
__global__ __launch_bounds__(kThreads, 1) void bwd_dkdv_kernel(Params p) {
  constexpr int BQ = 32 * NQB;           // queries per tile
  constexpr int ND = D / 16;             // reduction steps of S and dP
  constexpr int NMB = D / 32;            // 32-row blocks of dK^T, dV^T
  constexpr int CH = D / 8;              // 16-byte chunks per row
  constexpr int ROWB = D * 2;            // bytes per row
  constexpr int TILE = BQ * D;           // elements per Q (or dO) tile
  constexpr int TILEB = TILE * 2;
  constexpr int LPW = TILEB / 1024 / 4;  // 1 KB wave loads per tensor per wave
  constexpr int RPL = 1024 / ROWB;       // rows per 1 KB load
  constexpr int HB = D >= 128 ? 2 : 1;   // block flip of the +8-row half (see toff)
  static_assert(LPW * 4 * 1024 == TILEB && RPL >= 1, "tile split");
  static_assert(BQ * 4 <= 1024 && 64 % BQ == 0, "L/D vector load");

  // Stage s: Q tile at sm<s>[0], dO tile at sm<s>[TILE]; L log2 e and D
  // of the tile's rows at sv<s>[0] and sv<s>[BQ]. Separate arrays per stage
  // (selected at compile time) let the compiler see that reads of one stage
  // never wait for the loads still in flight into another.
  __shared__ __attribute__((aligned(1024))) bf16 sm0[2 * TILE];
  __shared__ __attribute__((aligned(1024))) bf16 sm1[2 * TILE];
  __shared__ __attribute__((aligned(1024))) bf16 sm2[2 * TILE];
  __shared__ __attribute__((aligned(1024))) bf16 sm3[2 * TILE];
  __shared__ __attribute__((aligned(16))) float sv0[2 * BQ];
  __shared__ __attribute__((aligned(16))) float sv1[2 * BQ];
  __shared__ __attribute__((aligned(16))) float sv2[2 * BQ];
  __shared__ __attribute__((aligned(16))) float sv3[2 * BQ];
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
        vf[kd] = as_bf16x8(kok ? (bb ^ 0x80008000u) : z);  // -V (see G above)
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
        *reinterpret_cast<u32x4*>(sm0 + e) = u32x4{0u, 0u, 0u, 0u};
        *reinterpret_cast<u32x4*>(sm1 + e) = u32x4{0u, 0u, 0u, 0u};
        *reinterpret_cast<u32x4*>(sm2 + e) = u32x4{0u, 0u, 0u, 0u};
        *reinterpret_cast<u32x4*>(sm3 + e) = u32x4{0u, 0u, 0u, 0u};
      }
      __syncthreads();  // the zeros land before any wave's tile loads
    }

    const int qsw = p.group;
    // The mask, applied branch-free on the masked steps (see below): a pair
    // (query q, key) is hidden iff q < qlo or q >= qhi, the queries that see
    // this lane's key (qlo = n for keys at or past the key limit). Query
    // tiles [tb, te) hold every query some key of the workgroup is seen by,
    // tiles [iu0, iu1) only queries that see all of its keys (the bounds are
    // non-decreasing in the key); rows past n are always masked.
    const Band<CAUSAL> band = make_band<CAUSAL>(p, n, kv_lim);
    const int qlo = band.qlo(mykey), qhi = band.qhi(mykey);
    const int k_last = min(k0 + kBKV, kv_lim) - 1;
    const int tb = band.qlo(k0) / BQ;
    const int te = (band.qhi(k_last) + BQ - 1) / BQ;
    const int iu0 = (band.qlo(k0 + kBKV - 1) + BQ - 1) / BQ;
    const int iu1 = band.qhi(k0) / BQ;

    // Loads of query tile it into a stage (sm: Q and dO, sv: L and D). Wave
    // w fills rows
    // [w * LPW * RPL, (w + 1) * LPW * RPL) of the Q and dO tiles; lane l of
    // a 1 KB load writes physical chunk l % CH of row l / CH, holding logical
    // chunk (l % CH) ^ swz_both(row). The descriptors span the head's n
    // rows, so rows past n are never read. Wave 0 also loads the tile's
    // L log2 e and D values (16 bytes per lane; the vectors are padded per
    // head to a multiple of 64 rows, so a tile is always in range).
    int ld_off[LPW];
#pragma unroll
    for (int i = 0; i < LPW; ++i) {
      const int row = (w * LPW + i) * RPL + lane / CH;
      ld_off[i] = (row * D + ((lane % CH) ^ swz_both<D>(row)) * 8) * 2;
    }
    // Per-lane LDS element offsets (tile-invariant). Row reads: row c of a
    // 32-row block, logical chunk kd*2 + h. Transposing reads: row
    // h*4 + (c%16)/4 of a 16-row block, column mb*32 + 16*(c/16) + 4*(c%4);
    // the second read of a fragment (rows +8) lands in block mb ^ HB.
    int qoff[ND], toff[NMB];
#pragma unroll
    for (int kd = 0; kd < ND; ++kd) qoff[kd] = c * D + (((kd * 2 + h) ^ swz_both<D>(c)) << 3);
    {
      const int trow = h * 4 + ((c & 15) >> 2);
      const int tcol = 16 * (c >> 4) + 4 * (c & 3);
#pragma unroll
      for (int mb = 0; mb < NMB; ++mb) {
        const int col = mb * 32 + tcol;
        toff[mb] = trow * D + (((col >> 3) ^ swz_both<D>(trow)) << 3) + (col & 7);
      }
    }

    auto sweep = [&](const auto& tiles) FA_INLINE {
    const int ns = tiles.count;
    if (ns == 0) return;
    for (int gq = 0; gq < qsw; ++gq) {
      // Query head gq of the group: its Q, dO and row vectors.
      // Work entry of query head hk * group + gq (workspace rows).
      const int bh = b * p.heads + hk * p.group + gq;
      const size_t base = span_row0(p, sp, p.heads, hk * p.group + gq) * D;
      const auto rq = buffer_rsrc(static_cast<const bf16*>(p.q) + base, n * ROWB);
      const auto rg = buffer_rsrc(static_cast<const bf16*>(p.d_o) + base, n * ROWB);
      const auto rl = buffer_rsrc(p.l2vec + (size_t)bh * p.n_pad, p.n_pad * 4);
      const auto rd = buffer_rsrc(p.dvec + (size_t)bh * p.n_pad, p.n_pad * 4);
      // Waves may still be reading the previous head's last tiles from the
      // stages; every wave is past them before they are refilled.
      if (gq > 0) __syncthreads();
      auto issue = [&](int it, bf16* sm, float* sv) FA_INLINE {
        const int qb0 = it * BQ * ROWB;
#pragma unroll
        for (int i = 0; i < LPW; ++i) {
          bload_lds16(rq, qb0 + ld_off[i], sm + (w * LPW + i) * RPL * D);
          bload_lds16(rg, qb0 + ld_off[i], sm + TILE + (w * LPW + i) * RPL * D);
        }
        if (w == 0 && lane < BQ / 4) {
          bload_lds16(rl, it * BQ * 4 + lane * 16, sv);
          bload_lds16_at(rd, it * BQ * 4 + lane * 16, sv, BQ * 4);
        }
      };

      // D of the tile in stage v in the accumulator layout of G: element
      // (gi, i) of block qb is query qb*32 + gi*8 + 4h + i.
      auto read_d = [&](const float* v, f32x16 (&dd)[NQB]) FA_INLINE {
#pragma unroll
        for (int qb = 0; qb < NQB; ++qb)
#pragma unroll
          for (int gi = 0; gi < 4; ++gi) {
            const f32x4 x = *reinterpret_cast<const f32x4*>(&v[BQ + qb * 32 + gi * 8 + h * 4]);
#pragma unroll
            for (int i = 0; i < 4; ++i) dd[qb][gi * 4 + i] = x[i];
          }
      };

      // S = Q K^T and G = D - dP (dO (-V)^T accumulated onto D) of the tile
      // in stage sm, D read from stage sv (lane = key, 16 queries per
      // 32-query block); used once per sweep, before the loop.
      auto sdp = [&](const bf16* sm, const float* sv, f32x16 (&s)[NQB], f32x16 (&g)[NQB]) FA_INLINE {
        f32x16 dd[NQB];
        read_d(sv, dd);
#pragma unroll
        for (int qb = 0; qb < NQB; ++qb) {
          s[qb] = mma32_v0(as_bf16x8(ld16(sm + qb * 32 * D + qoff[0])), kf[0]);
          g[qb] = mma32_vc(as_bf16x8(ld16(sm + TILE + qb * 32 * D + qoff[0])), vf[0], dd[qb]);
#pragma unroll
          for (int kd = 1; kd < ND; ++kd) {
            s[qb] = mma32_v(as_bf16x8(ld16(sm + qb * 32 * D + qoff[kd])), kf[kd], s[qb]);
            g[qb] = mma32_v(as_bf16x8(ld16(sm + TILE + qb * 32 * D + qoff[kd])), vf[kd], g[qb]);
          }
        }
        // dd stays live until every chain has moved past its first product.
#pragma unroll
        for (int qb = 0; qb < NQB; ++qb) keep_live(dd[qb], dd[qb]);
      };

      // P = exp2(S c - L log2 e) and -dS = P (D - dP) = P G for element e of
      // the lane's 16 NQB values, in place in s and g. Query of element
      // (qb, gi, i) is q0 + 4h + (qb*32 + gi*8 + i); the pair is hidden iff
      // that offset is < lo or >= hi, and a hidden pair gets P = 0, dS = 0.
      auto pds1 = [&](int e, int lo, int hi, const f32x4 (&l4)[NQB][4], f32x16 (&s)[NQB],
                      f32x16 (&g)[NQB], auto mask_tag) FA_INLINE {
        constexpr bool MASK = decltype(mask_tag)::value;
        const int qb = e / 16, r = e % 16, gi = r / 4, i = r % 4;
        const int off = qb * 32 + gi * 8 + i;
        const float x = (MASK && (off < lo || off >= hi)) ? kNegInf : s[qb][r];
        const float pr = __builtin_amdgcn_exp2f(fmaf(x, cs, -l4[qb][gi][i]));
        s[qb][r] = pr;
        g[qb][r] = pr * g[qb][r];
      };

      // A fragments of the transposing reads for (qb, qc, mb): dO^T and Q^T of
      // 16 queries x 32 dims of the tile in sm.
      auto trfrag = [&](const bf16* sm, int qb, int qc, int mb, bf16x8& fo, bf16x8& fq) FA_INLINE {
        const int r0 = (qb * 32 + qc * 16) * D;
        const int r1 = r0 + 8 * D;
        const u32x2 olo = ds_read_tr16(sm + TILE + r0 + toff[mb]);
        const u32x2 ohi = ds_read_tr16(sm + TILE + r1 + toff[mb ^ HB]);
        const u32x2 qlo = ds_read_tr16(sm + r0 + toff[mb]);
        const u32x2 qhi = ds_read_tr16(sm + r1 + toff[mb ^ HB]);
        fo = as_bf16x8(u32x4{olo[0], olo[1], ohi[0], ohi[1]});
        fq = as_bf16x8(u32x4{qlo[0], qlo[1], qhi[0], qhi[1]});
      };

      // One query tile, software-pipelined and issued in a fixed order (the
      // sched_barrier fences pin it): phase 1 computes S and G = D - dP of
      // tile it+1 (stage mB, row reads two products ahead; D from vB) into
      // sn, gn while the vector units turn S and G of tile it (in s, g; L
      // from vA) into P and -dS, 16/ND values per product pair; phase 2
      // accumulates dV^T and -dK^T of tile it from stage mA (transposing
      // reads one pair ahead). The next step takes sn, gn as its s, g.
      constexpr int NS = NQB * ND;        // phase-1 slots (2 products each)
      constexpr int EPS = 16 / ND;        // P/dS values per phase-1 slot
      constexpr int NP = NQB * 2 * NMB;   // phase-2 slots (2 products each)
      f32x16 sa[NQB], ga[NQB], sb[NQB], gb[NQB];
      auto body = [&](int it, const bf16* mA, const float* vA, const bf16* mB, const float* vB,
                      f32x16 (&s)[NQB], f32x16 (&g)[NQB], f32x16 (&sn)[NQB],
                      f32x16 (&gn)[NQB], auto mask_tag) FA_INLINE {
        const int qh = it * BQ + h * 4;
        const int lo = qlo - qh;
        const int hi = qhi - qh;
        f32x4 l4[NQB][4];
#pragma unroll
        for (int qb = 0; qb < NQB; ++qb)
#pragma unroll
          for (int gi = 0; gi < 4; ++gi)
            l4[qb][gi] = *reinterpret_cast<const f32x4*>(&vA[qb * 32 + gi * 8 + h * 4]);
        f32x16 dn[NQB];  // D of tile it+1: where its G chains start
        read_d(vB, dn);
        bf16x8 rq[3], rg[3];
#pragma unroll
        for (int j = 0; j < 2; ++j) {
          rq[j] = as_bf16x8(ld16(mB + (j / ND) * 32 * D + qoff[j % ND]));
          rg[j] = as_bf16x8(ld16(mB + TILE + (j / ND) * 32 * D + qoff[j % ND]));
        }
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int j = 0; j < NS; ++j) {
          {
            const int qb = j / ND, kd = j % ND;
            if (kd == 0) {
              sn[qb] = mma32_v0(rq[j % 3], kf[kd]);
              gn[qb] = mma32_vc(rg[j % 3], vf[kd], dn[qb]);
            } else {
              sn[qb] = mma32_v(rq[j % 3], kf[kd], sn[qb]);
              gn[qb] = mma32_v(rg[j % 3], vf[kd], gn[qb]);
            }
            if (j + 2 < NS) {
              const int j2 = j + 2;
              rq[j2 % 3] = as_bf16x8(ld16(mB + (j2 / ND) * 32 * D + qoff[j2 % ND]));
              rg[j2 % 3] = as_bf16x8(ld16(mB + TILE + (j2 / ND) * 32 * D + qoff[j2 % ND]));
            }
          }
#pragma unroll
          for (int e = j * EPS; e < (j + 1) * EPS; ++e) pds1(e, lo, hi, l4, s, g, mask_tag);
          __builtin_amdgcn_sched_barrier(0);
        }
        bf16x8 fo[2], fq[2];
        trfrag(mA, 0, 0, 0, fo[0], fq[0]);
        bf16x8 pfr, sfr;
#pragma unroll
        for (int k = 0; k < NP; ++k) {
          const int qb = k / (2 * NMB), qc = (k / NMB) % 2, mb = k % NMB;
          if (k + 1 < NP) {
            const int k1 = k + 1;
            trfrag(mA, k1 / (2 * NMB), (k1 / NMB) % 2, k1 % NMB, fo[k1 % 2], fq[k1 % 2]);
          }
          if (mb == 0) {
            u32x4 pu, su;
#pragma unroll
            for (int t = 0; t < 4; ++t) {
              pu[t] = pack_bf16x2(s[qb][qc * 8 + 2 * t], s[qb][qc * 8 + 2 * t + 1]);
              su[t] = pack_bf16x2(g[qb][qc * 8 + 2 * t], g[qb][qc * 8 + 2 * t + 1]);
            }
            pfr = as_bf16x8(pu);
            sfr = as_bf16x8(su);
          }
          dv[mb] = mma32(fo[k % 2], pfr, dv[mb]);
          dk[mb] = mma32(fq[k % 2], sfr, dk[mb]);
          __builtin_amdgcn_sched_barrier(0);
        }
        // sn, gn stay live to here even where nothing reads them (the last
        // tile's successor), and so does dn: otherwise the compiler may hand
        // their registers to other values while those products are still
        // writing (sn, gn) or reading (dn) them.
#pragma unroll
        for (int qb = 0; qb < NQB; ++qb) {
          keep_live(sn[qb], gn[qb]);
          keep_live(dn[qb], dn[qb]);
        }
      };

      // Step it uses stage it % 4 for tile it (A), stage (it + 1) % 4 for
      // tile it+1 (B) and sends tile it+2 to stage (it + 2) % 4 (C); the
      // scores of tile it are in register set it % 2. At the top of a step
      // each wave waits for its own loads of tile it+1; the barrier then
      // makes every wave's loads visible and guarantees that every wave has
      // finished the previous step, the last reader of stage C (tile it-2).
      auto step = [&](int it, auto stage_tag, auto mask_tag) FA_INLINE {
        constexpr int K = decltype(stage_tag)::value;
        bf16* const sms[4] = {sm0, sm1, sm2, sm3};
        float* const svs[4] = {sv0, sv1, sv2, sv3};
        wait_global_loads();
        __syncthreads();
        if (it + 2 < ns) issue(tiles.tile(it + 2), sms[(K + 2) % 4], svs[(K + 2) % 4]);
        if constexpr (K % 2 == 0)
          body(tiles.tile(it), sms[K], svs[K], sms[(K + 1) % 4], svs[(K + 1) % 4], sa, ga, sb, gb,
               mask_tag);
        else
          body(tiles.tile(it), sms[K], svs[K], sms[(K + 1) % 4], svs[(K + 1) % 4], sb, gb, sa, ga,
               mask_tag);
      };
      using S0 = std::integral_constant<int, 0>;
      using S1 = std::integral_constant<int, 1>;
      using S2 = std::integral_constant<int, 2>;
      using S3 = std::integral_constant<int, 3>;
      auto quad = [&](int it, auto mask_tag) FA_INLINE {
        step(it, S0{}, mask_tag);
        step(it + 1, S1{}, mask_tag);
        step(it + 2, S2{}, mask_tag);
        step(it + 3, S3{}, mask_tag);
      };

      // Steps (it counts steps; tiles.tile(it) is the query tile): masked
      // steps up to the first that holds only fully visible queries (the
      // causal diagonal band, or everything when the workgroup straddles the
      // key limit), rounded up to a multiple of four so the unmasked loop
      // starts with the same stage rotation; unmasked steps; masked steps
      // again (the window's far edge), the last step always among them (its
      // tile may be partial). The unmasked steps skip the mask arithmetic.
      const int last = ns - 1;
      const int su0 = tiles.first_at_least(iu0);
      const int su1 = tiles.first_at_least(iu1);
      const int head = min((su0 + 3) / 4 * 4, last);

      issue(tiles.tile(0), sm0, sv0);
      if (1 < ns) issue(tiles.tile(1), sm1, sv1);
      wait_global_loads();
      __syncthreads();
      sdp(sm0, sv0, sa, ga);
      int it = 0;
      for (; it + 4 <= head; it += 4) quad(it, std::true_type{});
      // Here either it == head with it % 4 == 0, or head == last and fewer
      // than four steps remain before it, so the loops below do not run.
      for (; it + 4 <= min(su1, last); it += 4) quad(it, std::false_type{});
      for (; it + 4 <= last; it += 4) quad(it, std::true_type{});
      // last - it is 0 to 3 here: one masked step per remaining tile. The
      // step of the last tile also computes S and dP of a successor that does
      // not exist, from the finite data left in its stage, and drops them
      // (one tile's two products per sweep): a separate finishing body needs
      // registers of its own and made the compiler spill the accumulators.
      step(it, S0{}, std::true_type{});
      if (it + 1 <= last) {
        step(it + 1, S1{}, std::true_type{});
        if (it + 2 <= last) {
          step(it + 2, S2{}, std::true_type{});
          if (it + 3 <= last) step(it + 3, S3{}, std::true_type{});
        }
      }
    }  // query heads of the group
    };
    if constexpr (SPARSE) {
      // The workgroup's 128 keys are one block column of the mask.
      const int nl = stage_blocks(col_blocks(p, k0 / kBlock), sblk, tid, kThreads, p.nb);
      sweep(sparse_tiles<kBlock / BQ>(sblk, nl, tb, te));
    } else {
      sweep(dense_tiles(tb, te));
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

template <int D, int NQB>
hipError_t launch_d(const Params& p, hipStream_t s) {
  const int t_c = (p.n + kBKV - 1) / kBKV;
  const long long total = (long long)t_c * p.batch * p.heads_kv;
  dim3 grid((unsigned)total), block(kThreads);
  return dispatch_mask(p, [&](auto causal, auto sparse) {
    hipLaunchKernelGGL((bwd_dkdv_kernel<D, NQB, decltype(causal)::value, decltype(sparse)::value>),
                       grid, block, 0, s, p);
    return hipGetLastError();
  });
}

}  // namespace

hipError_t launch_bwd_dkdv_bf16(const Params& p, int d, hipStream_t s) {
  switch (d) {
    // d = 64: sequences up to 1024 rows go to the 16-key kernel of
    // fa_bwd_dkdv_d64.hip, whose higher occupancy wins when many short key
    // tiles share the chip; for longer ones the busiest workgroup's serial
    // sweep sets the time, and this kernel's pipelined waves run it faster.
    case 64: return p.n <= 1024 ? launch_bwd_dkdv_bf16_d64(p, d, s) : launch_d<64, 2>(p, s);
    // 64 keys per wave (fa_bwd_dkdv_wide.hip) from 4096 rows, without a
    // block mask or a window; shorter sequences leave too few of its 256-key
    // workgroups to fill the GPU.
    case 128:
      return p.blk == nullptr && p.win_left < 0 && p.win_right < 0 && p.n >= 4096
                 ? launch_bwd_dkdv_bf16_wide(p, d, s)
                 : launch_d<128, 1>(p, s);
    case 256: return launch_bwd_dkdv_bf16_d256(p, d, s);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace fa
