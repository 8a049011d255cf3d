// Attention backward, dK/dV part, for d = 64 and sequences of at most 1024
// rows: bf16 in/out, fp32 accumulate, for gfx950 (the other shapes use
// fa_bwd_bf16.hip and fa_bwd_dkdv_d256.hip).
//
// Method: recomputation from the saved row statistic (page 1, "注意力为什么
// 受限于显存带宽：用算术强度与分块把 FlashAttention 推导清楚", section 八; page 2,
// "4. FlashAttention 深度剖析", 4.3.4): P_ij = exp(scale q_i.k_j - L_i) is
// rebuilt tile by tile and never stored; with dP = dO V^T and
// D_i = <dO_i, O_i> (formed by the dQ kernel, which runs first),
//     dV = P^T dO,  dS = P * (dP - D),  dK = scale dS^T Q.
// As in fa_bwd_bf16.hip, G = D - dP is formed on the matrix cores (dO (-V)^T
// accumulated onto D) and P * G = -dS is accumulated, so dK is scaled by
// -scale at the end.
//
// Mapping onto CDNA4. A workgroup is 4 wave64s (one per SIMD) and owns 64
// keys, 16 per wave, with their dK, dV accumulators (fp32) for the whole
// query sweep (key/value-outer order: each written once, no atomics). The
// products are v_mfma_f32_16x16x32_bf16 (16 x 16 results, reduction 32):
// * S = Q K^T and G = D + dO (-V)^T per 16-query block: A = Q (dO) rows read
//   from LDS, B = the wave's K (-V) rows held in registers; the result holds
//   one key per lane (lane % 16) and queries 4 (lane / 16) + 0..3.
// * dV^T += dO^T P and dK^T += Q^T (P G) per 16-channel block: the B operand
//   is P (P G) of 32 queries, which a lane already holds -- queries
//   {4g .. 4g + 3, 16 + 4g .. 16 + 4g + 3} (g = lane / 16) of its key --
//   packed to bf16; the A operand dO^T (Q^T) for those queries is two
//   transposing LDS reads (ds_read_b64_tr_b16) of the row-major tile.
// Compared with one wave per SIMD holding 32 keys (fa_bwd_bf16.hip), a wave
// needs half the accumulator and K/V registers (128 VGPRs in all), so four
// workgroups share a CU, four waves per SIMD, and each hides the others'
// waits; in exchange each A operand read from LDS feeds 16 keys instead of
// 32, twice the LDS reads per product. That trade wins where many short key
// tiles share the chip (d = 64, up to 1024 rows); on long sequences it is
// even or slower, and at d = 128 (204 VGPRs, two waves per SIMD) the doubled
// LDS reads make it slower than the 32-key kernel throughout.
//
// Query tiles (BQ rows of Q and dO, and their L log2 e and D values) go from
// HBM straight into LDS through buffer descriptors, row-major with the XOR
// swizzle swz16 that keeps both the row reads and the transposing reads
// conflict-free; two stages, the next tile loading during the current step,
// one barrier per step.
#include <type_traits>

#include "fa_device.h"

namespace fa {

namespace {

constexpr int kThreads = 256;
constexpr int kBKV = 64;  // keys per workgroup (4 waves x 16)

// acc[16x16] += A[16x32] B[32x16] on the bf16 matrix cores, fp32 accumulate.
// Lane l supplies row (l % 16) of A and column (l % 16) of B, each with 8
// reduction indices chosen by l / 16 (any assignment works as long as A and
// B use it alike). The result holds column (l % 16), rows 4 (l / 16) + 0..3.
__device__ __forceinline__ f32x4 mma16(bf16x8 a, bf16x8 b, f32x4 acc) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, acc, 0, 0, 0);
}

// XOR swizzle of the 16-byte chunk index within a tile row (64 bf16, no
// padding; a row covers half the LDS banks, so rows of one parity share a
// half), a function of t = (row >> 1) % 8. Two access patterns read the
// tile: row reads (ds_read_b128; lane l reads row l % 16 at logical chunk
// 4 kd + l / 16) and transposing reads (ds_read_b64_tr_b16; lane l reads
// 8 bytes of row 4 (l / 16) + (l % 16) / 4 at a 32-byte column block). The
// swizzle keeps both free of bank conflicts whichever lanes the LDS serves
// together in one pass: for row reads 16 consecutive lanes, lanes 8p..8p+7
// with 32+8p..32+8p+7 (the grouping the conflict counter points to: the
// simpler swizzle ((t % 4) << 1) | (t / 4), conflict-free for consecutive
// lanes, measured 0.28 conflict cycles per LDS cycle), or four lanes of
// each 16; for transposing reads 32 or 16 consecutive lanes, or 16 of each
// half-wave. It was found by exhaustive search over the bijections of t
// with a host model of both patterns.
__device__ __forceinline__ int swz16(int row) {
  const int t = (row >> 1) & 7;
  return ((t & 1) << 2) | ((((t >> 1) ^ (t >> 2)) & 1) << 1) | ((t >> 1) & 1);
}

template <bool CAUSAL, bool SPARSE>
// (Four workgroups per CU: the compiler keeps the kernel within 128
// registers per lane.)
__global__ __launch_bounds__(kThreads, 4) void bwd_dkdv_d64_kernel(Params p) {
  constexpr int D = 64;
  constexpr int BQ = 64;                  // queries per tile (one 1 KB load per wave per tensor)
  constexpr int NQ16 = BQ / 16;           // 16-query blocks of S and G
  constexpr int NQK = BQ / 32;            // 32-query reduction steps of dV, dK
  constexpr int NKD = D / 32;             // 32-channel reduction steps of S and G
  constexpr int NDB = D / 16;             // 16-channel blocks of dK^T, dV^T
  constexpr int CH = D / 8;               // 16-byte chunks per row
  constexpr int ROWB = D * 2;             // bytes per row
  constexpr int TILE = BQ * D;            // elements per Q (or dO) tile
  constexpr int NW = kThreads / 64;
  constexpr int RPL = 1024 / ROWB;        // rows per 1 KB load
  constexpr int LPW = TILE * 2 / 1024 / NW;  // 1 KB loads per wave per tensor
  static_assert(LPW * NW * 1024 == TILE * 2, "tile split");
  static_assert(BQ * 4 <= 16 * 64, "L/D vector load");

  // Stage s: Q tile at sm<s>[0], dO tile at sm<s>[TILE]; L log2 e and D of
  // the tile's rows at sv<s>[0] and sv<s>[BQ].
  __shared__ __attribute__((aligned(1024))) bf16 sm0[2 * TILE];
  __shared__ __attribute__((aligned(1024))) bf16 sm1[2 * TILE];
  __shared__ __attribute__((aligned(16))) float sv0[2 * BQ];
  __shared__ __attribute__((aligned(16))) float sv1[2 * BQ];
  __shared__ int sblk[SPARSE ? kMaxBlocks : 1];

  const int tid = threadIdx.x;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lane = tid & 63;
  const int m = lane & 15;  // key of the lane (results), row of A / column of B
  const int g = lane >> 4;  // reduction group (operands), result row group

  const int t_c = (p.n + kBKV - 1) / kBKV;
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
  const int kw0 = k0 + w * 16;
  const int mykey = kw0 + m;
  const float cs = p.c;
  // A negative scale is applied by negating K (exact in bf16): the scores
  // use K' = -K with |scale|, and dK = scale dS^T Q with the true Q.
  const uint32_t kflip = p.q_neg ? 0x80008000u : 0u;

  f32x4 dk[NDB], dv[NDB];
#pragma unroll
  for (int db = 0; db < NDB; ++db) {
    dk[db] = f32x4{};
    dv[db] = f32x4{};
  }

  if (k0 < kv_lim) {
    // K and -V rows of this lane's key as B fragments: [mykey][kd*32 + 8g + e].
    // Keys past the key limit are read clamped and replaced by zeros.
    bf16x8 kf[NKD], vf[NKD];
    {
      const bool kok = mykey < kv_lim;
      const int kr = kok ? mykey : kv_lim - 1;
#pragma unroll
      for (int kd = 0; kd < NKD; ++kd) {
        const u32x4 z = {0u, 0u, 0u, 0u};
        const u32x4 a = ld16(K + (size_t)kr * D + kd * 32 + g * 8);
        const u32x4 bb = ld16(V + (size_t)kr * D + kd * 32 + g * 8);
        kf[kd] = as_bf16x8(kok ? (a ^ kflip) : z);
        vf[kd] = as_bf16x8(kok ? (bb ^ 0x80008000u) : z);
      }
    }

    // Stages start as zeros: out-of-range lanes of a partial tile may leave
    // their LDS bytes as they were, and a masked row must hold finite data.
    {
      constexpr int NZ = 2 * TILE * 2 / 16 / kThreads;
      static_assert(NZ * 16 * kThreads == 2 * TILE * 2, "zero fill");
#pragma unroll
      for (int t = 0; t < NZ; ++t) {
        const int e = (t * kThreads + tid) * 8;
        *reinterpret_cast<u32x4*>(sm0 + e) = u32x4{0u, 0u, 0u, 0u};
        *reinterpret_cast<u32x4*>(sm1 + e) = u32x4{0u, 0u, 0u, 0u};
      }
      __syncthreads();
    }

    // Masks: the pair (query q, key) is hidden iff q < qlo or q >= qhi, the
    // queries that see this lane's key. Query tiles [tb, te) hold every
    // query some key of the workgroup is seen by, tiles [iu0, iu1) only
    // queries that see all of its keys; [wqlo, wqhi) the queries some key of
    // this wave is seen by (a masked tile outside it is skipped).
    const Band<CAUSAL> band = make_band<CAUSAL>(p, n, kv_lim);
    const int qlo = band.qlo(mykey), qhi = band.qhi(mykey);
    const int k_last = min(k0 + kBKV, kv_lim) - 1;
    const int tb = band.qlo(k0) / BQ;
    const int te = (band.qhi(k_last) + BQ - 1) / BQ;
    const int iu0 = (band.qlo(k0 + kBKV - 1) + BQ - 1) / BQ;
    const int iu1 = band.qhi(k0) / BQ;
    const int wqlo = band.qlo(kw0);
    const int wqhi = band.qhi(min(kw0 + 15, kv_lim - 1));

    // Tile loads: wave w fills rows [w*LPW*RPL, (w+1)*LPW*RPL) of the Q and
    // dO tiles, one 1 KB load per RPL rows; lane l writes physical chunk
    // l % CH of row l / CH, holding logical chunk (l % CH) ^ swz16(row).
    int ld_off[LPW];
#pragma unroll
    for (int i = 0; i < LPW; ++i) {
      const int ld_row = (w * LPW + i) * RPL + lane / CH;
      ld_off[i] = (ld_row * D + ((lane % CH) ^ swz16(ld_row)) * 8) * 2;
    }
    // Operand offsets (elements, tile-invariant). Row reads (A of S, G): row
    // qb*16 + m, logical chunk kd*4 + g. Transposing reads (A of dV^T, dK^T):
    // lane addresses row 4g + (m >> 2) (+16 for the second read), column
    // db*16 + 4 (m & 3), and receives rows 4g + 0..3 of column db*16 + m.
    int roff[NKD];
#pragma unroll
    for (int kd = 0; kd < NKD; ++kd) roff[kd] = m * D + (((kd * 4 + g) ^ swz16(m)) << 3);
    // (The swizzle repeats every 16 rows, so the second read of a fragment
    // is the first one 16 rows further on: a constant offset.)
    const int trow = 4 * g + (m >> 2);
    int toff[NDB];
#pragma unroll
    for (int db = 0; db < NDB; ++db) {
      const int col = db * 16 + 4 * (m & 3);
      toff[db] = trow * D + (((col >> 3) ^ swz16(trow)) << 3) + (col & 7);
    }

    auto sweep = [&](const auto& tiles) FA_INLINE {
      const int ns = tiles.count;
      if (ns == 0) return;
      const int su0 = tiles.first_at_least(iu0);
      const int su1 = max(tiles.first_at_least(iu1), su0);
      for (int gq = 0; gq < p.group; ++gq) {
        // Query head gq of the group: its Q, dO and row vectors.
        const int bh = b * p.heads + hk * p.group + gq;
        const size_t base = span_row0(p, sp, p.heads, hk * p.group + gq) * D;
        const auto rq = buffer_rsrc(static_cast<const bf16*>(p.q) + base, n * ROWB);
        const auto rg = buffer_rsrc(static_cast<const bf16*>(p.d_o) + base, n * ROWB);
        const auto rl = buffer_rsrc(p.l2vec + (size_t)bh * p.n_pad, p.n_pad * 4);
        const auto rd = buffer_rsrc(p.dvec + (size_t)bh * p.n_pad, p.n_pad * 4);
        // Waves may still be reading the previous head's last tiles.
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
        // One query tile (stage sm, sv): S and G, then P and P G, then the
        // dV^T and dK^T products.
        auto compute = [&](int it, const bf16* sm, const float* sv, auto mask_tag) FA_INLINE {
          constexpr bool MASK = decltype(mask_tag)::value;
          f32x4 s[NQ16], gg[NQ16];
#pragma unroll
          for (int qb = 0; qb < NQ16; ++qb) {
            // G's chain starts from the D values of the block's queries.
            gg[qb] = *reinterpret_cast<const f32x4*>(&sv[BQ + qb * 16 + 4 * g]);
            s[qb] = f32x4{};
#pragma unroll
            for (int kd = 0; kd < NKD; ++kd) {
              const bf16x8 aq = as_bf16x8(ld16(sm + qb * 16 * D + roff[kd]));
              const bf16x8 ag = as_bf16x8(ld16(sm + TILE + qb * 16 * D + roff[kd]));
              s[qb] = mma16(aq, kf[kd], s[qb]);
              gg[qb] = mma16(ag, vf[kd], gg[qb]);
            }
          }
          // P = exp2(S c - L log2 e) and P G = -dS; hidden pairs get P = 0.
          const int qh = it * BQ + 4 * g;
          bf16x8 pfr[NQK], sfr[NQK];
#pragma unroll
          for (int qk = 0; qk < NQK; ++qk) {
            u32x4 pu, su;
#pragma unroll
            for (int half = 0; half < 2; ++half) {
              const int qb = 2 * qk + half;
              const f32x4 l4 = *reinterpret_cast<const f32x4*>(&sv[qb * 16 + 4 * g]);
              float pr[4], ds[4];
#pragma unroll
              for (int i = 0; i < 4; ++i) {
                float x = s[qb][i];
                if (MASK) {
                  const int q = qh + qb * 16 + i;
                  x = (q < qlo || q >= qhi) ? kNegInf : x;
                }
                pr[i] = __builtin_amdgcn_exp2f(fmaf(x, cs, -l4[i]));
                ds[i] = pr[i] * gg[qb][i];
              }
              pu[2 * half] = pack_bf16x2(pr[0], pr[1]);
              pu[2 * half + 1] = pack_bf16x2(pr[2], pr[3]);
              su[2 * half] = pack_bf16x2(ds[0], ds[1]);
              su[2 * half + 1] = pack_bf16x2(ds[2], ds[3]);
            }
            pfr[qk] = as_bf16x8(pu);
            sfr[qk] = as_bf16x8(su);
          }
#pragma unroll
          for (int qk = 0; qk < NQK; ++qk)
#pragma unroll
            for (int db = 0; db < NDB; ++db) {
              const int r0 = qk * 32 * D;
              const u32x2 o0 = ds_read_tr16(sm + TILE + r0 + toff[db]);
              const u32x2 o1 = ds_read_tr16(sm + TILE + r0 + 16 * D + toff[db]);
              const u32x2 q0 = ds_read_tr16(sm + r0 + toff[db]);
              const u32x2 q1 = ds_read_tr16(sm + r0 + 16 * D + toff[db]);
              dv[db] = mma16(as_bf16x8(u32x4{o0[0], o0[1], o1[0], o1[1]}), pfr[qk], dv[db]);
              dk[db] = mma16(as_bf16x8(u32x4{q0[0], q0[1], q1[0], q1[1]}), sfr[qk], dk[db]);
            }
        };
        // Two stages, one barrier per step: at the top of step m this wave
        // waits for its own loads of the step's tile, the barrier makes every
        // wave's loads visible and guarantees every wave has finished step
        // m-1, whose stage is then refilled with the next tile. A masked
        // tile none of this wave's keys is seen by is skipped.
        auto iter = [&](int mm, const bf16* sm, const float* sv, bf16* nsm, float* nsv,
                        auto mask_tag) FA_INLINE {
          constexpr bool MASK = decltype(mask_tag)::value;
          const int it = tiles.tile(mm);
          wait_global_loads();
          __syncthreads();
          if (mm + 1 < ns) issue(tiles.tile(mm + 1), nsm, nsv);
          if (MASK && (it * BQ >= wqhi || it * BQ + BQ <= wqlo)) return;
          compute(it, sm, sv, mask_tag);
        };
        auto gen = [&](int mm, const bf16* sm, const float* sv, bf16* nsm, float* nsv) FA_INLINE {
          if (mm >= su0 && mm < su1) iter(mm, sm, sv, nsm, nsv, std::false_type{});
          else iter(mm, sm, sv, nsm, nsv, std::true_type{});
        };
        issue(tiles.tile(0), sm0, sv0);
        // Whole pairs before the unmasked steps, unmasked pairs, then the
        // rest (a last single step only in the final loop).
        int mm = 0;
        for (; mm < su0 && mm + 1 < ns; mm += 2) {
          gen(mm, sm0, sv0, sm1, sv1);
          gen(mm + 1, sm1, sv1, sm0, sv0);
        }
        for (; mm + 1 < su1; mm += 2) {
          iter(mm, sm0, sv0, sm1, sv1, std::false_type{});
          iter(mm + 1, sm1, sv1, sm0, sv0, std::false_type{});
        }
        for (; mm < ns; mm += 2) {
          gen(mm, sm0, sv0, sm1, sv1);
          if (mm + 1 >= ns) break;
          gen(mm + 1, sm1, sv1, sm0, sv0);
        }
      }  // query heads of the group
    };
    if constexpr (SPARSE) {
      // The workgroup's 64 keys lie in one block column of the mask.
      const int nl = stage_blocks(col_blocks(p, k0 / kBlock), sblk, tid, kThreads, p.nb);
      sweep(sparse_tiles<kBlock / BQ>(sblk, nl, tb, te));
    } else {
      sweep(dense_tiles(tb, te));
    }
  }

  // dK = scale * (dS^T Q) (dk holds -dS^T Q), dV as accumulated; lane's key
  // mykey, channels db*16 + 4g + 0..3.
  if (mykey < n) {
    const float ks = -p.scale;
#pragma unroll
    for (int db = 0; db < NDB; ++db) {
      const size_t off = (size_t)mykey * D + db * 16 + 4 * g;
      u32x2 uk, uv;
      uk[0] = pack_bf16x2(dk[db][0] * ks, dk[db][1] * ks);
      uk[1] = pack_bf16x2(dk[db][2] * ks, dk[db][3] * ks);
      uv[0] = pack_bf16x2(dv[db][0], dv[db][1]);
      uv[1] = pack_bf16x2(dv[db][2], dv[db][3]);
      *reinterpret_cast<u32x2*>(dK + off) = uk;
      *reinterpret_cast<u32x2*>(dV + off) = uv;
    }
  }
}

}  // namespace

hipError_t launch_bwd_dkdv_bf16_d64(const Params& p, int d, hipStream_t s) {
  if (d != 64) return hipErrorInvalidValue;
  const int t_c = (p.n + kBKV - 1) / kBKV;
  const long long total = (long long)t_c * p.batch * p.heads_kv;
  dim3 grid((unsigned)total), block(kThreads);
  return dispatch_mask(p, [&](auto causal, auto sparse) {
    hipLaunchKernelGGL((bwd_dkdv_d64_kernel<decltype(causal)::value, decltype(sparse)::value>),
                       grid, block, 0, s, p);
    return hipGetLastError();
  });
}

}  // namespace fa
