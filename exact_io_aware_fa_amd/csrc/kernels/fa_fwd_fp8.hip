// Attention forward on FP8 (E4M3) operands with fp32 accumulation, for
// gfx950 (d = 64, 128 and 256).
//
// Method: page 2 ("4. FlashAttention 深度剖析"), 4.5.4 (FP8 support): both
// products of the forward take E4M3 operands, every block carries the scale
// it was encoded with, and the products accumulate in fp32. The tiling and
// the (m, l, O) update are those of the bf16 forward (page 2 4.3.2; page 1,
// "注意力为什么受限于显存带宽：用算术强度与分块把 FlashAttention 推导清楚",
// section 六), with two changes the format asks for:
// * the running row reference is an integer frame f = ceil(max t) in base-2
//   units (t = s * c), so every rescale factor 2^(f_old - f_new) is a power
//   of two: a probability rounded in an earlier, lower frame is the same
//   E4M3 value as if it had been rounded in the final frame (in the normal
//   range), whatever the tile order;
// * probabilities enter the P V product as E4M3(2^(t - f + 8)), in (0, 256]:
//   the factor 2^8 moves the largest probabilities of a row to the top of the
//   format's normal range (<= 448); l is the sum of the rounded values, so
//   O = O~ / l weights the V rows by exactly the probabilities the product
//   used, and the 2^8 cancels.
//
// Operands (written by the quantiser kernel):
// * Q, K codes row-major [rows][d] bytes; the scores of a tile are
//   (Q K^T codes) * sigma_q * sigma_k, the two block scales folded into the
//   exp2 factor (c_j = |scale| log2(e) sigma_q sigma_k,j);
// * V codes stored per 128-key block transposed ([d channels][128 keys]);
//   the V block scale is a power of two and enters the P V product through
//   the matrix core's own E8M0 operand scale, so O~ needs no rescale when
//   the V block changes.
//
// Mapping onto CDNA4 (as the bf16 forward): 8 wave64s per workgroup, 256
// query rows, 32 per wave for the whole key sweep; ping-pong between the
// two waves of a SIMD (matrix phase of one, softmax phase of the other).
// At d = 256 a wave's O accumulator alone is 128 registers, which with the
// Q codes and the score tile exceeds the 256 registers a wave may hold when
// two share a SIMD: there the workgroup is 4 waves (128 rows, one wave per
// SIMD with up to 512 registers), each running both phases in turn;
// K and V^T tiles straight from HBM into LDS (two stages each). The score
// product is S^T = K Q^T on v_mfma_f32_32x32x64_f8f6f4: lane l supplies
// query l % 32 as B and key row sigma(l % 32) as A, with
// sigma(8a + 4b + i) = 16b + 4a + i, so that the result register r of lane
// (c, h) holds key 16h + r of its 32-key block: each lane then owns 16
// consecutive keys per block, and its rounded probabilities are directly
// the B operand of O^T += V^T P^T, whose A operand (V^T) is read as two
// 16-byte runs of one channel row.
#include <float.h>

#include <type_traits>

#include "fa_device.h"

namespace fa {

namespace {

typedef int i32x8 __attribute__((ext_vector_type(8)));

// acc[32x32] += A[32x64] B[64x32] on the E4M3 matrix cores, fp32 accumulate.
// Lane l supplies row l % 32 of A and column l % 32 of B, each with 32 of
// the 64 reduction indices (chosen by l / 32); byte k of an A lane pairs
// with byte k of the B lane of the same half, so any assignment of
// reduction indices to bytes works as long as A and B use it alike. Result
// layout as mma32. mma_f8_s scales A by 2^(sa - 127) and B by 2^(sb - 127)
// (E8M0 bytes, per lane: lane l's scale applies to the 32 reduction indices
// it supplies of row / column l % 32).
__device__ __forceinline__ f32x16 mma_f8(i32x8 a, i32x8 b, f32x16 acc) {
  return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, acc, 0, 0, 0, 0, 0, 0);
}
__device__ __forceinline__ f32x16 mma_f8_s(i32x8 a, i32x8 b, f32x16 acc, int sa, int sb) {
  return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, acc, 0, 0, 0, sa, 0, sb);
}

__device__ __forceinline__ float halves_max(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x),
                                                  false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}

// Key row read by A lane c of a 32-key block (see the header).
__device__ __forceinline__ int key_of_lane(int c) {
  return 16 * ((c >> 2) & 1) + 4 * (c >> 3) + (c & 3);
}
// XOR swizzles of the 16-byte chunk index. K rows (d bytes): the 16 lanes
// of a read phase touch rows {0..7, 16..23} (or {8..15, 24..31}) of a block
// at one logical chunk; rows that share bank groups (same parity for
// 128-byte rows, same row % 4 for 64-byte rows) must land on different
// chunks, which these swizzles do. V^T rows (BC bytes): 16 consecutive rows
// at one logical chunk.
// (256-byte rows all start at bank 0: the 16 rows of a phase take 16
// different chunks.)
template <int D>
__device__ __forceinline__ int swz_k(int row) {
  if (D == 256) return (row & 7) | ((row >> 1) & 8);
  return D == 128 ? (((row >> 1) & 3) | ((row >> 2) & 4)) : (((row >> 2) & 1) | ((row >> 3) & 2));
}
template <int BC>
__device__ __forceinline__ int swz_v(int row) {
  return BC == 64 ? ((row >> 2) & 3) : ((row >> 1) & 7);
}

// A wave-uniform float loaded by every lane with a vector load (so that it
// is counted by vmcnt, like the tile loads, and not by lgkmcnt, like the LDS
// reads of the matrix phase).
__device__ __forceinline__ float vload_uniform(const float* a, int i) {
  int z = 0;
  asm volatile("" : "+v"(z));
  return a[i + z];
}

template <int D, int BC, bool CAUSAL, int NWAVES>
__global__ __launch_bounds__(NWAVES * 64, 1) void fwd_fp8_kernel(Fp8Params p) {
  // 8 waves: ping-pong between waves w and w + 4 (groups A and B); 4 waves:
  // every wave is in group A and runs both phases of each step.
  constexpr int kThreads = NWAVES * 64;
  constexpr int kBR = 32 * NWAVES;       // query rows per workgroup
  static_assert(NWAVES == 8 || NWAVES == 4, "workgroup shape");
  constexpr int NQF = D / 64;            // 64-channel halves of a score product
  constexpr int CPR = D / 16;            // 16-byte chunks per K row
  constexpr int TILEB = BC * D;          // bytes of a K or V^T tile
  constexpr int NW = kThreads / 64;      // waves per workgroup
  constexpr int LPW = TILEB / 1024 / NW;  // 1 KB loads per tensor per wave
  constexpr int KRPL = 1024 / D;         // K rows per 1 KB load
  constexpr int VCH = BC / 16;           // 16-byte chunks per V^T row
  constexpr int VRPL = 1024 / BC;        // V^T rows per 1 KB load
  constexpr int NKB = BC / 32;           // 32-key blocks of S^T
  constexpr int NKK = BC / 64;           // 64-key reduction chunks of O^T
  constexpr int NMB = D / 32;            // 32-channel blocks of O^T
  static_assert(LPW >= 1 && LPW * NW * 1024 == TILEB, "tile split");
  static_assert(BC == 64 || BC == 128, "tile width");
  static_assert(D == 64 || D == 128 || D == 256, "head dim");

  __shared__ __attribute__((aligned(1024))) uint8_t sK0[TILEB];
  __shared__ __attribute__((aligned(1024))) uint8_t sK1[TILEB];
  __shared__ __attribute__((aligned(1024))) uint8_t sV0[TILEB];
  __shared__ __attribute__((aligned(1024))) uint8_t sV1[TILEB];

  const int tid = threadIdx.x;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int grp = NWAVES == 8 ? (w >> 2) : 0;
  const int lane = tid & 63;
  const int c = lane & 31;
  const int h = lane >> 5;

  const int n = p.n;
  const int t_r = (n + kBR - 1) / kBR;
  int b, hq, qb;
  remap_workgroup(blockIdx.x, gridDim.x, t_r, CAUSAL, p.batch, b, hq, qb);
  const size_t bhq = (size_t)b * p.heads + hq;
  const size_t bhk = (size_t)b * p.heads_kv + hq / p.group;
  const uint8_t* __restrict__ Q8 = p.q8 + bhq * (size_t)p.np * D;
  const uint8_t* __restrict__ K8 = p.k8 + bhk * (size_t)p.np * D;
  const uint8_t* __restrict__ V8 = p.v8 + bhk * (size_t)p.np * D;
  const float* __restrict__ ksc = p.k_scale + bhk * p.nb;
  const float* __restrict__ vsc = p.v_scale + bhk * p.nb;
  bf16* __restrict__ O = static_cast<bf16*>(p.o) + bhq * (size_t)n * D;

  int kv_lim = n;
  if (p.kv_len != nullptr) kv_lim = min(max(p.kv_len[b], 0), n);
  const int q0 = qb * kBR;
  const int qw0 = NWAVES == 8 ? q0 + 32 * (2 * (w & 3) + grp) : q0 + 32 * w;
  const int qi = qw0 + c;
  // exp2 factor of this wave's rows: |scale| log2(e) sigma_q (one block).
  const float cq = p.c * p.q_scale[bhq * p.nb + min(qw0 / 128, p.nb - 1)];

  // Q codes of this wave's rows as B fragments: lane (c, h) holds bytes
  // 64 kd + 32 h .. + 31 of row qi. A negative scale negates the codes
  // (sign bit, exact); rows past n are zero.
  i32x8 qf[NQF];
  {
    const uint32_t flip = p.q_neg ? 0x80808080u : 0u;
    const int qr = min(qi, n - 1);
#pragma unroll
    for (int kd = 0; kd < NQF; ++kd) {
      const uint8_t* src = Q8 + (size_t)qr * D + kd * 64 + h * 32;
      const u32x4 lo = ld16(src) ^ flip, hi = ld16(src + 16) ^ flip;
      const bool in = qi < n;
      qf[kd] = i32x8{(int)(in ? lo[0] : 0u), (int)(in ? lo[1] : 0u), (int)(in ? lo[2] : 0u),
                     (int)(in ? lo[3] : 0u), (int)(in ? hi[0] : 0u), (int)(in ? hi[1] : 0u),
                     (int)(in ? hi[2] : 0u), (int)(in ? hi[3] : 0u)};
    }
  }

  // Key ranges as in the bf16 forward (no window: every row starts at key
  // 0, so the masked steps of a wave are the last ones).
  const Band<CAUSAL> band{n, kv_lim, -1, -1};
  const int ntiles = max((band.hi(min(q0 + kBR, n) - 1) + BC - 1) / BC, 0);
  const int qw_last = min(qw0 + 31, n - 1);
  const int s_first = 0;
  const int s_last = (band.hi(qw_last) - 1) / BC;
  const int su_hi = band.hi(qw0) / BC;

  f32x16 acc[NMB];
#pragma unroll
  for (int mb = 0; mb < NMB; ++mb) acc[mb] = f32x16{};
  // Row sums l = sum_j P^_j on the matrix cores: the product of an all-ones
  // A operand with the P^T fragments gives every row of this block the sum
  // over the tile's keys (both reduction halves), in the same frame as O~.
  f32x16 accl = f32x16{};
  float f = kNegInf;   // integer frame of the running row max (base-2 units)
  float fo = kNegInf;  // frame of the accumulators O~ and l: the row's first frame
  f32x16 sc[NKB];
  i32x8 pf[NKK];
  int sb = 127;        // E8M0 scale 2^(f - fo) of the pending P^T fragments
#pragma unroll
  for (int kk = 0; kk < NKK; ++kk) pf[kk] = i32x8{0, 0, 0, 0, 0, 0, 0, 0};

  // DMA offsets (tile-invariant). K: lane l of load i writes physical chunk
  // l % 8 of row (w LPW + i) 8 + l / 8, fetching logical chunk
  // (l % CPR) ^ swz_k(row). V^T: row (w LPW + i) VRPL + l / VCH, chunk l % VCH.
  int ld_koff[LPW], ld_voff[LPW];
#pragma unroll
  for (int i = 0; i < LPW; ++i) {
    const int kr = (w * LPW + i) * KRPL + lane / CPR;
    ld_koff[i] = kr * D + (((lane % CPR) ^ swz_k<D>(kr)) << 4);
    const int vr = (w * LPW + i) * VRPL + lane / VCH;
    ld_voff[i] = vr * 128 + (((lane % VCH) ^ swz_v<BC>(vr)) << 4);
  }
  auto issue_k = [&](int j, uint8_t* dst) FA_INLINE {
    const auto r = buffer_rsrc(K8 + (size_t)j * BC * D, TILEB);
#pragma unroll
    for (int i = 0; i < LPW; ++i) bload_lds16(r, ld_koff[i], dst + (w * LPW + i) * 1024);
  };
  auto issue_v = [&](int j, uint8_t* dst) FA_INLINE {
    const int kb0 = j * BC;
    const auto r =
        buffer_rsrc(V8 + (size_t)(kb0 >> 7) * (D * 128) + (kb0 & 127), D * 128 - (kb0 & 127));
#pragma unroll
    for (int i = 0; i < LPW; ++i) bload_lds16(r, ld_voff[i], dst + (w * LPW + i) * 1024);
  };

  // Operand read offsets (tile-invariant): K row key_of_lane(c) of each
  // 32-key block, logical chunks 4 kd + 2 h + {0, 1}; V^T row c of each
  // 32-channel block, logical chunks 4 kk + h and 4 kk + 2 + h.
  int koff[NQF][2], voff[NKK][2];
  {
    const int kr = key_of_lane(c);
#pragma unroll
    for (int kd = 0; kd < NQF; ++kd)
#pragma unroll
      for (int e = 0; e < 2; ++e)
        koff[kd][e] = kr * D + (((4 * kd + 2 * h + e) ^ swz_k<D>(kr)) << 4);
#pragma unroll
    for (int kk = 0; kk < NKK; ++kk)
#pragma unroll
      for (int e = 0; e < 2; ++e)
        voff[kk][e] = c * BC + (((4 * kk + 2 * e + h) ^ swz_v<BC>(c)) << 4);
  }

  // Matrix phase: S^T slots (NKB blocks x 2 halves of d), then O^T slots
  // (NMB channel blocks x NKK key chunks), operands read PF slots ahead.
  constexpr int NS = NKB * NQF;
  constexpr int NPV = NMB * NKK;
  constexpr int PF = 3;
  auto rd = [&](const uint8_t* sk, const uint8_t* sv, int k) FA_INLINE {
    u32x4 lo, hi;
    if (k < NS) {
      const int kb = k % NKB, kd = k / NKB;
      const uint8_t* base = sk + kb * 32 * D;
      lo = ld16(base + koff[kd][0]);
      hi = ld16(base + koff[kd][1]);
    } else {
      const int mb = (k - NS) % NMB, kk = (k - NS) / NMB;
      const uint8_t* base = sv + mb * 32 * BC;
      lo = ld16(base + voff[kk][0]);
      hi = ld16(base + voff[kk][1]);
    }
    return i32x8{(int)lo[0], (int)lo[1], (int)lo[2], (int)lo[3],
                 (int)hi[0], (int)hi[1], (int)hi[2], (int)hi[3]};
  };
  auto slots = [&](const uint8_t* sk, const uint8_t* sv, int ve) FA_INLINE {
#pragma unroll
    for (int kb = 0; kb < NKB; ++kb) sc[kb] = f32x16{};
    i32x8 fr[PF + 1];
#pragma unroll
    for (int k = 0; k < PF; ++k) fr[k] = rd(sk, sv, k);
#pragma unroll
    for (int k = 0; k < NS + NPV; ++k) {
      if (k + PF < NS + NPV) fr[(k + PF) % (PF + 1)] = rd(sk, sv, k + PF);
      if (k < NS) {
        const int kb = k % NKB, kd = k / NKB;
        sc[kb] = mma_f8(fr[k % (PF + 1)], qf[kd], sc[kb]);
      } else {
        const int mb = (k - NS) % NMB, kk = (k - NS) / NMB;
        acc[mb] = mma_f8_s(fr[k % (PF + 1)], pf[kk], acc[mb], ve, sb);
      }
      __builtin_amdgcn_sched_barrier(0);
    }
    constexpr int kOnes = 0x38383838;  // four E4M3 1.0
#pragma unroll
    for (int kk = 0; kk < NKK; ++kk) {
      accl = mma_f8_s(i32x8{kOnes, kOnes, kOnes, kOnes, kOnes, kOnes, kOnes, kOnes}, pf[kk],
                      accl, 127, sb);
      __builtin_amdgcn_sched_barrier(0);
    }
    // Keep the products in this half-period: otherwise the compiler sinks
    // the O^T products past the next barrier, next to their first use.
    // (Ping-pong only: with one wave per SIMD there is nothing to overlap,
    // and the accumulators may live in AGPRs.)
    if constexpr (NWAVES == 8) {
#pragma unroll
      for (int mb = 0; mb < NMB; ++mb) asm volatile("" : "+v"(acc[mb]));
      asm volatile("" : "+v"(accl));
    }
  };

  // Softmax phase of tile j with exp2 factor cj.
  auto apply_mask = [&](int j) FA_INLINE {
    const int kb0 = j * BC;
    int qv = qi;
    asm volatile("" : "+v"(qv));
    const int hi_i = band.hi(qv);
#pragma unroll
    for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int key = kb0 + kb * 32 + 16 * h + r;
        sc[kb][r] = key >= hi_i ? kNegInf : sc[kb][r];
      }
  };
  auto softmax = [&](float cj) FA_INLINE {
    float mp[4] = {kNegInf, kNegInf, kNegInf, kNegInf};
#pragma unroll
    for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
      for (int r = 0; r < 16; ++r) mp[r & 3] = fmaxf(mp[r & 3], sc[kb][r]);
    const float mt = halves_max(fmaxf(fmaxf(mp[0], mp[1]), fmaxf(mp[2], mp[3])));
    // New integer frame: ceil of the running max of t = s * cj (cj > 0, so
    // -inf stays -inf). Probabilities are rounded in this frame.
    const float fnew = fmaxf(f, ceilf(mt * cj));
    f = fnew;
    const float fref = (fnew == kNegInf) ? 0.f : fnew;
    const float off = 8.f - fref;
#pragma unroll
    for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
      for (int r = 0; r < 16; ++r) sc[kb][r] = __builtin_amdgcn_exp2f(fmaf(sc[kb][r], cj, off));
    // O~ and l stay in the row's first frame fo: this tile's contribution
    // enters scaled by 2^(f - fo), a power of two that the P V product (and
    // the row-sum product) applies through its B-operand scale, so the
    // accumulators are never rescaled. Only when the gap would leave the
    // safe exponent range (scores spread over more than 2^64) are they moved
    // to the current frame.
    fo = (fo == kNegInf) ? fnew : fo;
    if (__builtin_amdgcn_ballot_w64(fnew - fo > 64.f)) {
      const float alpha = __builtin_amdgcn_exp2f(fo - fref);
#pragma unroll
      for (int mb = 0; mb < NMB; ++mb) acc[mb] *= alpha;
      accl *= alpha;
      fo = fnew;
    }
    sb = 127 + ((fnew == kNegInf) ? 0 : (int)(fnew - fo));
    // P^T fragments: bytes 0-15 from block 2 kk, 16-31 from block 2 kk + 1,
    // four probabilities per dword (RNE to E4M3).
#pragma unroll
    for (int kk = 0; kk < NKK; ++kk)
#pragma unroll
      for (int q = 0; q < 8; ++q) {
        const f32x16& v = sc[2 * kk + (q >> 2)];
        const int r = 4 * (q & 3);
        uint32_t w8 = __builtin_amdgcn_cvt_pk_fp8_f32(v[r], v[r + 1], 0u, false);
        w8 = __builtin_amdgcn_cvt_pk_fp8_f32(v[r + 2], v[r + 3], w8, true);
        pf[kk][q] = (int)w8;
      }
    if constexpr (NWAVES == 8) {
#pragma unroll
      for (int kk = 0; kk < NKK; ++kk) asm volatile("" : "+v"(pf[kk]));
      asm volatile("" : "+v"(sb));
    }
  };
  auto valu_phase = [&](int j, float cj) FA_INLINE {
    if (j >= 0 && j < ntiles && j >= s_first && j <= s_last) {
      if (j >= su_hi) apply_mask(j);
      softmax(cj);
    } else {
#pragma unroll
      for (int kk = 0; kk < NKK; ++kk) pf[kk] = i32x8{0, 0, 0, 0, 0, 0, 0, 0};
      sb = 127;
    }
  };

  // Per-tile scales, loaded one step ahead with the tiles: at step m the
  // softmax of tile m (group A) uses cj_m, that of tile m - 1 (group B)
  // cj_m1, and the P V product of tile m - 1 uses V exponent ve_m1.
  auto kfactor = [&](int j) FA_INLINE {
    return vload_uniform(ksc, min(j * BC / 128, p.nb - 1));
  };
  auto vexp = [&](int j) FA_INLINE {
    return vload_uniform(vsc, min(j * BC / 128, p.nb - 1));
  };
  float k_nx = kfactor(0);  // sigma_k of tile m + 1 (in flight)
  float v_nx = 1.f;         // sigma_v of tile m (in flight); tile -1: P is 0
  float cj_m = 0.f, cj_m1 = 0.f;
  int ve_m1 = 127;

  auto phase_barrier = [&]() FA_INLINE {
    __builtin_amdgcn_sched_barrier(0);
    __syncthreads();
    __builtin_amdgcn_sched_barrier(0);
  };
  auto mid_barrier = [&]() FA_INLINE {
    __builtin_amdgcn_sched_barrier(0);
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_sched_barrier(0);
  };
  auto open_step = [&](int m, uint8_t* nk, uint8_t* nv) FA_INLINE {
    wait_global_loads();
    // The scale loads of the previous step have landed: take them over
    // before this step's loads are issued.
    asm volatile("" : "+v"(k_nx), "+v"(v_nx));
    cj_m1 = cj_m;
    cj_m = fmaxf(cq * k_nx, FLT_MIN);
    ve_m1 = (int)((__float_as_uint(v_nx) >> 23) & 0xFF);
    phase_barrier();
    if (m + 1 < ntiles) {
      issue_k(m + 1, nk);
      k_nx = kfactor(m + 1);
    }
    if (m < ntiles) {
      issue_v(m, nv);
      v_nx = vexp(m);
    }
  };
  auto step_a = [&](int m, const uint8_t* sk, uint8_t* nk, uint8_t* nv, const uint8_t* sv)
      FA_INLINE {
    open_step(m, nk, nv);
    slots(sk, sv, ve_m1);
    mid_barrier();
    valu_phase(m, cj_m);
  };
  auto step_b = [&](int m, const uint8_t* sk, uint8_t* nk, uint8_t* nv, const uint8_t* sv)
      FA_INLINE {
    open_step(m, nk, nv);
    valu_phase(m - 1, cj_m1);
    mid_barrier();
    slots(sk, sv, ve_m1);
  };
  auto hot_a = [&](int m, const uint8_t* sk, uint8_t* nk, uint8_t* nv, const uint8_t* sv)
      FA_INLINE {
    open_step(m, nk, nv);
    slots(sk, sv, ve_m1);
    mid_barrier();
    softmax(cj_m);
  };
  auto hot_b = [&](int m, const uint8_t* sk, uint8_t* nk, uint8_t* nv, const uint8_t* sv)
      FA_INLINE {
    open_step(m, nk, nv);
    softmax(cj_m1);
    mid_barrier();
    slots(sk, sv, ve_m1);
  };

  // All stages start zeroed (finite data under masked or unused rows).
  {
    constexpr int NZ = TILEB / 16 / kThreads;
    static_assert(NZ * 16 * kThreads == TILEB, "zero fill");
#pragma unroll
    for (int t = 0; t < NZ; ++t) {
      const int e = (t * kThreads + tid) * 16;
      *reinterpret_cast<u32x4*>(sK0 + e) = u32x4{0u, 0u, 0u, 0u};
      *reinterpret_cast<u32x4*>(sK1 + e) = u32x4{0u, 0u, 0u, 0u};
      *reinterpret_cast<u32x4*>(sV0 + e) = u32x4{0u, 0u, 0u, 0u};
      *reinterpret_cast<u32x4*>(sV1 + e) = u32x4{0u, 0u, 0u, 0u};
    }
    __syncthreads();
  }

  // Steps as in the bf16 forward: whole pairs from step 1 with fixed stage
  // assignments; steps [1, hot_end) take the straight-line steps.
  const int hot_end = min(min(ntiles, s_last + 1), su_hi + grp);
  if (ntiles > 0) issue_k(0, sK0);
  if (grp == 0) {
    step_a(0, sK0, sK1, sV0, sV1);
    int m = 1;
    for (; m + 1 < hot_end; m += 2) {
      hot_a(m, sK1, sK0, sV1, sV0);
      hot_a(m + 1, sK0, sK1, sV0, sV1);
    }
    for (; m <= ntiles; m += 2) {
      step_a(m, sK1, sK0, sV1, sV0);
      if (m + 1 > ntiles) break;
      step_a(m + 1, sK0, sK1, sV0, sV1);
    }
  } else {
    step_b(0, sK0, sK1, sV0, sV1);
    int m = 1;
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

  // Epilogue: O = O~ / l (bf16), LSE = ln 2 (fo - 8 + log2 l).
  const float l = accl[0];
  if (qi < n) {
    const float inv = l > 0.f ? 1.f / l : 0.f;
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
    if (h == 0) p.lse[bhq * n + qi] = l > 0.f ? (fo - 8.f + __log2f(l)) * kLn2 : kNegInf;
  }
}

template <int D>
hipError_t launch_d(const Fp8Params& p, hipStream_t s) {
  constexpr int NW = D == 256 ? 4 : 8;
  constexpr int BR = 32 * NW;
  const int t_r = (p.n + BR - 1) / BR;
  const long long total = (long long)t_r * p.batch * p.heads;
  dim3 grid((unsigned)total), block(NW * 64);
  // 128-key tiles: half the per-tile overhead of 64 (barriers, row max
  // exchange, frame update) for the same matrix work.
  constexpr int BC = 128;
  if (p.causal)
    hipLaunchKernelGGL((fwd_fp8_kernel<D, BC, true, NW>), grid, block, 0, s, p);
  else
    hipLaunchKernelGGL((fwd_fp8_kernel<D, BC, false, NW>), grid, block, 0, s, p);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_fwd_fp8(const Fp8Params& p, int d, hipStream_t s) {
  switch (d) {
    case 64: return launch_d<64>(p, s);
    case 128: return launch_d<128>(p, s);
    case 256: return launch_d<256>(p, s);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace fa
