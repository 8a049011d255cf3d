// Device-side helpers shared by the gfx950 attention kernels: vector types,
// the bf16 matrix-core product, bf16 packing, and the workgroup-id remap.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

#include "../fa_internal.h"

namespace fa {

typedef __bf16 bf16;
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

// For lambdas inside kernels: a call that is not inlined would pass the
// captured state through memory, which costs registers, scratch traffic and
// the knowledge that values are wave-uniform.
#define FA_INLINE __attribute__((always_inline))

constexpr float kNegInf = -__builtin_inff();
constexpr float kLn2 = 0.693147180559945309f;
constexpr float kLog2e = 1.442695040888963407f;

// acc[32x32] += A[32x16] * B[16x32] on the bf16 matrix cores, fp32 accumulate.
// Lane l supplies row (l % 32) of A and column (l % 32) of B, each with the
// same 8 reduction indices, so any bijection between (l / 32, element) and
// the 16 reduction indices gives the same product as long as A and B use
// it alike. The result holds column (l % 32) and rows
// 8 * (r / 4) + 4 * (l / 32) + (r % 4), r = 0..15.
__device__ __forceinline__ f32x16 mma32(bf16x8 a, bf16x8 b, f32x16 acc) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, acc, 0, 0, 0);
}

// v_mfma_f32_32x32x16_bf16 with its accumulator in VGPRs, as inline
// assembly: for kernels where the compiler would give its matrix builtins
// the AGPR form (more than 256 registers per lane in play), so that vector
// code can read the results without a v_accvgpr_read each. The compiler's
// hazard tracking does not see these products; the caller must keep every
// result and accumulator input untouched until the product is done (about
// a dozen wait states for this 8-pass product: mfma_drain, or enough other
// instructions) and must not place two products of one chain back to back
// unless the second accumulates onto exactly the first's result.
// mma32_v accumulates onto c in place; mma32_v0 starts a chain at zero;
// mma32_vc starts one at c, into new registers. A result may not overlap
// the A, B or C registers (they are still read while it is written): hence
// the early-clobber outputs. A vector instruction that writes an operand
// needs two wait states before a product reads it; the compiler inserts
// them for its own products only, so a kernel using these forms must not
// let one come closer (the ISA hazard test checks the generated code of
// every kernel that uses them). The w forms (mma32_vw, mma32_v0w, mma32_vcw) open with
// the two wait states themselves, for kernels where the register allocator
// brings operands back from AGPRs right before the products.
__device__ __forceinline__ f32x16 mma32_v(bf16x8 a, bf16x8 b, f32x16 c) {
  asm volatile("v_mfma_f32_32x32x16_bf16 %0, %1, %2, %0" : "+v"(c) : "v"(a), "v"(b));
  return c;
}
__device__ __forceinline__ f32x16 mma32_v0(bf16x8 a, bf16x8 b) {
  f32x16 d;
  asm volatile("v_mfma_f32_32x32x16_bf16 %0, %1, %2, 0" : "=&v"(d) : "v"(a), "v"(b));
  return d;
}
__device__ __forceinline__ f32x16 mma32_vc(bf16x8 a, bf16x8 b, const f32x16& c) {
  f32x16 d;
  asm volatile("v_mfma_f32_32x32x16_bf16 %0, %1, %2, %3" : "=&v"(d) : "v"(a), "v"(b), "v"(c));
  return d;
}
__device__ __forceinline__ f32x16 mma32_vw(bf16x8 a, bf16x8 b, f32x16 c) {
  asm volatile("s_nop 1\n\tv_mfma_f32_32x32x16_bf16 %0, %1, %2, %0" : "+v"(c) : "v"(a), "v"(b));
  return c;
}
__device__ __forceinline__ f32x16 mma32_v0w(bf16x8 a, bf16x8 b) {
  f32x16 d;
  asm volatile("s_nop 1\n\tv_mfma_f32_32x32x16_bf16 %0, %1, %2, 0" : "=&v"(d) : "v"(a), "v"(b));
  return d;
}
__device__ __forceinline__ f32x16 mma32_vcw(bf16x8 a, bf16x8 b, const f32x16& c) {
  f32x16 d;
  asm volatile("s_nop 1\n\tv_mfma_f32_32x32x16_bf16 %0, %1, %2, %3"
               : "=&v"(d) : "v"(a), "v"(b), "v"(c));
  return d;
}
// An empty use of two values in VGPRs (keeps them, and their registers,
// live up to this point).
__device__ __forceinline__ void keep_live(const f32x16& x, const f32x16& y) {
  asm volatile("" ::"v"(x), "v"(y));
}
// 20 wait states: enough for any result of the products above to be
// written before the next instruction reads it.
__device__ __forceinline__ void mfma_drain() {
  __builtin_amdgcn_sched_barrier(0);
  asm volatile("s_nop 15\n\ts_nop 3" ::: "memory");
  __builtin_amdgcn_sched_barrier(0);
}

__device__ __forceinline__ bf16x8 as_bf16x8(u32x4 v) {
  return __builtin_bit_cast(bf16x8, v);
}

__device__ __forceinline__ u32x4 ld16(const void* p) {
  return *reinterpret_cast<const u32x4*>(p);
}

__device__ __forceinline__ u32x2 ld8(const void* p) {
  return *reinterpret_cast<const u32x2*>(p);
}

// Round to nearest even, two floats -> one dword of two bf16 (low = a).
__device__ __forceinline__ uint32_t pack_bf16x2(float a, float b) {
  typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
  bf16x2 r;
  r[0] = (__bf16)a;
  r[1] = (__bf16)b;
  return __builtin_bit_cast(uint32_t, r);
}

// Column e (0..7) of four 8-element bf16 rows, packed as 4 bf16 (row 0 in
// the lowest half-word): one 8-byte group of a transposed tile. One byte
// permute per output dword: selector 0x05040100 takes the low half-words of
// (src1, src0), 0x07060302 the high ones.
__device__ __forceinline__ u32x2 column4(const u32x4 r[4], int e) {
  const int w = e >> 1;
  const uint32_t sel = (e & 1) ? 0x07060302u : 0x05040100u;
  u32x2 out;
  out[0] = __builtin_amdgcn_perm(r[1][w], r[0][w], sel);
  out[1] = __builtin_amdgcn_perm(r[3][w], r[2][w], sel);
  return out;
}

// ---------------------------------------------------------------------------
// LDS helpers for tiles loaded straight from HBM into LDS.
//
// gload_lds16: 16 bytes from global address g (per lane) into LDS at
// lds_base + 16 * lane; lds_base must be the same for the whole wave. The
// data lands asynchronously and is tracked by vmcnt.
typedef __attribute__((address_space(3))) void lds_void;

__device__ __forceinline__ void gload_lds16(const void* g, void* lds_base) {
  __builtin_amdgcn_global_load_lds(g, (lds_void*)lds_base, 16, 0, 0);
}

// Buffer resource for `bytes` bytes from base (raw buffer: stride 0, data
// format word of the gfx9 family). base and bytes must be wave-uniform, so the
// descriptor lives in scalar registers. Loads through it at byte offsets at or
// past `bytes` are out of range: they read no memory and return zero.
// (The size goes through readfirstlane: a clamp such as max(min(x, a), 0)
// becomes a vector instruction, and a descriptor word in a vector register
// makes the compiler wrap every load in a loop over the lanes.)
__device__ __forceinline__ __amdgpu_buffer_rsrc_t buffer_rsrc(const void* base, int bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0,
                                           __builtin_amdgcn_readfirstlane(bytes), 0x00020000);
}

// bload_lds16: 16 bytes at byte offset voff (per lane) of a buffer into LDS
// at lds_base + 16 * lane, like gload_lds16 but with a 32-bit lane offset
// and range checking by the descriptor.
__device__ __forceinline__ void bload_lds16(__amdgpu_buffer_rsrc_t r, int voff, void* lds_base) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_void*)lds_base, 16, voff, 0, 0, 0);
}

// bload_lds16 into LDS at lds_base + lds_off bytes, the offset applied after
// the cast to the LDS address space. (A constant offset applied to the
// generic pointer of a __shared__ array first leaves a constant cast that the
// gfx950 instruction selector rejects when it sits inside a loop.)
__device__ __forceinline__ void bload_lds16_at(__amdgpu_buffer_rsrc_t r, int voff, void* lds_base,
                                               int lds_off) {
  typedef __attribute__((address_space(3))) char lds_char;
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_void*)((lds_char*)lds_base + lds_off), 16,
                                           voff, 0, 0, 0);
}

// Wait until this wave's outstanding global loads (including the loads into
// LDS) have completed; other counters are left alone. Encoding for gfx9:
// vmcnt = 0, expcnt = 7 (no wait), lgkmcnt = 15 (no wait).
__device__ __forceinline__ void wait_global_loads() { __builtin_amdgcn_s_waitcnt(0x0F70); }

// Transposing LDS read (ds_read_b64_tr_b16). Within each group of 16 lanes,
// lane i receives element (i % 4) of the 8-byte chunks addressed by lanes
// 4j + i/4 (j = 0..3) of its group. With a row-major bf16 tile and lane
// (c, h) = (lane % 32, lane / 32) pointing at
//     tile[r0 + 4h + (c % 16) / 4][d0 + 16 * (c / 16) + 4 * (c % 4)],
// lane (c, h) receives tile[r0 + 4h + j][d0 + c] for j = 0..3: four rows of
// one column, i.e. a transposed 8-byte MFMA operand fragment.
__device__ __forceinline__ u32x2 ds_read_tr16(const void* lds_addr) {
  typedef short s16x4 __attribute__((ext_vector_type(4)));
  const s16x4 v = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
      (__attribute__((address_space(3))) s16x4*)lds_addr);
  return __builtin_bit_cast(u32x2, v);
}

// XOR swizzles of the 16-byte chunk index within a tile row (rows of D bf16,
// no padding), chosen so that both access patterns hit every LDS bank once
// per 256 bytes:
// * row reads (lane c reads 16 bytes of row c): rows r..r+15 must map a given
//   chunk to 16 different bank groups;
// * transposing reads (a half-wave reads 4 rows x 64 bytes): the 4 rows'
//   chunk blocks must not overlap.
template <int D>
__device__ __forceinline__ int swz_row(int row) {
  return D >= 128 ? (row & 15) : ((row >> 1) & 7);
}
template <int D>
__device__ __forceinline__ int swz_tr(int row) {
  return D >= 128 ? 4 * (row & 3) : 4 * ((row >> 1) & 1);
}

// One swizzle serving both patterns on the same tile: it is a bijection on
// any 16 consecutive rows (same parity for d = 64) and moves any 4
// consecutive rows (from a multiple of 4) to 4 different 64-byte blocks.
template <int D>
__device__ __forceinline__ int swz_both(int row) {
  if (D >= 128) return (row & 15) ^ ((row & 3) << 2);
  const int v = (row >> 1) & 7;
  return v ^ ((v & 1) << 2);
}

// Workgroup remap. The dispatcher places consecutive workgroup ids on the
// eight XCDs in turn (id % 8), each XCD with its own L2. Hand each XCD a
// contiguous range of the work list, ordered head-major, then by tile, with
// the batch entry fastest: an XCD then holds a block of heads for every batch
// entry (the same work per XCD even when the entries of a packed batch have
// very different lengths), and within a head the tiles run from the most
// expensive down (largest work first). `tile` counts down from the last tile
// when `heavy_last_index` is set (causal forward: the last query tile sees
// the most keys), else up from tile 0 (causal backward: the first key tile
// sees the most queries).
__device__ __forceinline__ void remap_workgroup(int wg, int total, int tiles,
                                                bool heavy_last_index, int batch,
                                                int& b, int& head, int& tile) {
  const int xcd = wg & 7;
  const int slot = wg >> 3;
  const int per = total >> 3;
  const int rem = total & 7;
  const int idx = xcd * per + (xcd < rem ? xcd : rem) + slot;
  const int ht = idx / batch;  // head * tiles + t
  b = idx - ht * batch;
  head = ht / tiles;
  const int t = ht - head * tiles;
  tile = heavy_last_index ? (tiles - 1 - t) : t;
}

// Grouped K/V heads: query head h uses K/V head h / group (contiguous
// groups of `group` query heads share one K/V head).

// Rows of batch entry b: start .. start + len - 1 of each head of memory
// batch mb (see Params). The offsets of a packed batch are clamped so that
// every row lies inside the head's rows, whatever the device array holds.
struct Span {
  int start;
  int len;
  int mb;
};
__device__ __forceinline__ Span batch_span(const Params& p, int b) {
  if (p.cu_seqlens == nullptr) return Span{0, p.n, b};
  int a = p.cu_seqlens[b];
  int e = p.cu_seqlens[b + 1];
  a = a < 0 ? 0 : (a > p.rows ? p.rows : a);
  e = e < a ? a : (e > p.rows ? p.rows : e);
  const int len = e - a;
  return Span{a, len < p.n ? len : p.n, 0};
}
// Index of the first row of entry s in head hh of a tensor with nh heads.
__device__ __forceinline__ size_t span_row0(const Params& p, const Span& s, int nh, int hh) {
  return ((size_t)s.mb * nh + hh) * (size_t)p.rows + s.start;
}

// The backward's row terms, formed by the query-outer dQ kernel for its own
// rows and written to the workspace for the dK/dV kernel, which runs after
// it: D_i = <dO_i, O_i> in fp32 (the row term of dS = P * (dP - D); softmax
// calculus gives sum_j P_ij dP_ij = <dO_i, O_i>) and L_i log2(e), the saved
// row statistic in base-2 units (+inf for a row with no visible key, so that
// every rebuilt probability of it is exactly 0). Lane (c, h) holds elements
// kd*16 + h*8 .. +7 of its row's dO as fragments gf[kd] and reads the same
// elements of O from orow; the two halves of the row are summed with
// v_permlane32_swap (the same sum on both lanes). Rows [len, n_pad) of the
// entry get 0 and 0 (they are loaded, never used).
template <int ND>
__device__ __forceinline__ void bwd_row_terms(const Params& p, int bh, int qi, int len,
                                              const bf16* orow, const bf16x8 (&gf)[ND],
                                              float lse, int h, float& dd, float& l2) {
  float s = 0.f;
#pragma unroll
  for (int kd = 0; kd < ND; ++kd) {
    const u32x4 o = ld16(orow + kd * 16 + h * 8);
    const u32x4 g = __builtin_bit_cast(u32x4, gf[kd]);
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      s = fmaf(__uint_as_float(o[j] << 16), __uint_as_float(g[j] << 16), s);
      s = fmaf(__uint_as_float(o[j] & 0xffff0000u), __uint_as_float(g[j] & 0xffff0000u), s);
    }
  }
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(s), __float_as_uint(s), false,
                                                  false);
  dd = __uint_as_float(r[0]) + __uint_as_float(r[1]);
  l2 = lse == kNegInf ? __builtin_inff() : lse * kLog2e;
  if (h == 0 && qi < p.n_pad) {
    const size_t row = (size_t)bh * p.n_pad + qi;
    p.dvec[row] = qi < len ? dd : 0.f;
    p.l2vec[row] = qi < len ? l2 : 0.f;
  }
}

// Keys j >= kv_limit are hidden for batch entry b of length n (clamped to
// [0, n]).
__device__ __forceinline__ int kv_limit(const Params& p, int b, int n) {
  if (p.kv_len == nullptr) return n;
  int v = p.kv_len[b];
  v = v < 0 ? 0 : v;
  return v > n ? n : v;
}

// Interval masks -- causal, key padding and the sliding window -- of one
// batch entry of length n. Query row i (0-based in its entry) sees keys
// [lo(i), hi(i)); key j is seen by queries [qlo(j), qhi(j)). All four bounds
// are non-decreasing, so the first and last row (key) of a tile bound the
// whole tile. A window side of -1 is unbounded.
template <bool CAUSAL>
struct Band {
  int n, kv_lim, wl, wr;
  __device__ __forceinline__ int lo(int i) const { return wl >= 0 ? max(i - wl, 0) : 0; }
  __device__ __forceinline__ int hi(int i) const {
    int h = kv_lim;
    if (CAUSAL) h = min(h, i + 1);
    if (wr >= 0) h = min(h, i + wr + 1);
    return h;
  }
  __device__ __forceinline__ int qlo(int j) const {
    if (j >= kv_lim) return n;
    int l = CAUSAL ? j : 0;
    if (wr >= 0) l = max(l, j - wr);
    return l;
  }
  __device__ __forceinline__ int qhi(int j) const { return wl >= 0 ? min(n, j + wl + 1) : n; }
};
template <bool CAUSAL>
__device__ __forceinline__ Band<CAUSAL> make_band(const Params& p, int n, int kv_lim) {
  return Band<CAUSAL>{n, kv_lim, p.win_left, p.win_right};
}

// Block-sparse index (built by the index kernel from a block mask over
// kBlock x kBlock blocks, nb per side): row_ptr[nb + 1], col_idx[nb * nb],
// col_ptr[nb + 1], row_idx[nb * nb] -- for query block r the visible key
// blocks col_idx[row_ptr[r] .. row_ptr[r + 1]), for key block c the query
// blocks row_idx[col_ptr[c] .. col_ptr[c + 1]), both ascending.
constexpr int kBlock = 128;
constexpr int kMaxBlocks = 1024;  // nb limit: the list of one row fits LDS
struct BlockList {
  const int32_t* idx;
  int count;
};
// The list of row r (column c). Offsets and counts are clamped to the index's
// extent, so a malformed index cannot send a kernel out of bounds.
__device__ __forceinline__ BlockList clamp_list(const int32_t* ptr, const int32_t* idx, int i,
                                                int nb) {
  const int a = min(max(ptr[i], 0), nb * nb);
  const int e = min(max(ptr[i + 1], a), nb * nb);
  return BlockList{idx + a, min(e - a, nb)};
}
__device__ __forceinline__ BlockList row_blocks(const Params& p, int r) {
  return clamp_list(p.blk, p.blk + (p.nb + 1), r, p.nb);
}
__device__ __forceinline__ BlockList col_blocks(const Params& p, int c) {
  const int32_t* cp = p.blk + (p.nb + 1) + p.nb * p.nb;
  return clamp_list(cp, cp + (p.nb + 1), c, p.nb);
}
// Copies a block list into LDS (every thread of the workgroup takes part; a
// barrier follows) and returns its length. Entries are clamped to [0, nb).
__device__ __forceinline__ int stage_blocks(BlockList l, int* lds, int tid, int nthreads, int nb) {
  for (int i = tid; i < l.count; i += nthreads) lds[i] = min(max(l.idx[i], 0), nb - 1);
  __syncthreads();
  return l.count;
}

// The tiles a workgroup visits, in ascending order, as a function of the
// step number m in [0, count). Dense: the tiles [tb, te). Sparse: the tiles
// of the listed blocks (TPB tiles each) that fall inside [tb, te).
struct DenseTiles {
  int t0, count;
  // (readfirstlane: the value is wave-uniform anyway, and an opaque step
  // keeps the compiler from strength-reducing every address derived from the
  // tile into a register of its own across the loop.)
  __device__ __forceinline__ int tile(int m) const {
    return __builtin_amdgcn_readfirstlane(t0 + m);
  }
  // First step whose tile is >= x (count if none).
  __device__ __forceinline__ int first_at_least(int x) const { return min(max(x - t0, 0), count); }
  // Steps [s0, s1) of the tiles in [lo, hi).
  __device__ __forceinline__ void steps_of(int lo, int hi, int& s0, int& s1) const {
    s0 = first_at_least(lo);
    s1 = max(first_at_least(hi), s0);
  }
};
__device__ __forceinline__ DenseTiles dense_tiles(int tb, int te) {
  return DenseTiles{tb, max(te - tb, 0)};
}
template <int TPB>
struct SparseTiles {
  const int* lst;  // LDS: ascending block indices
  int nent;        // entries in lst
  int s;           // tiles of the first block before tb (skipped)
  int count;
  __device__ __forceinline__ int tile(int m) const {
    const int k = m + s;
    return lst[k / TPB] * TPB + k % TPB;
  }
  __device__ __forceinline__ int first_at_least(int x) const {
    int a = 0, e = nent;  // first entry whose last tile is >= x
    while (a < e) {
      const int mid = (a + e) >> 1;
      if (lst[mid] * TPB + TPB - 1 >= x) e = mid; else a = mid + 1;
    }
    if (a == nent) return count;
    const int m = a * TPB + max(x - lst[a] * TPB, 0) - s;
    return min(max(m, 0), count);
  }
  __device__ __forceinline__ void steps_of(int lo, int hi, int& s0, int& s1) const {
    s0 = first_at_least(lo);
    s1 = max(first_at_least(hi), s0);
  }
};
// The same tiles from the last one down (step m visits tile count-1-m).
template <class T>
struct ReversedTiles {
  T up;
  int count;
  __device__ __forceinline__ int tile(int m) const { return up.tile(count - 1 - m); }
  __device__ __forceinline__ void steps_of(int lo, int hi, int& s0, int& s1) const {
    int a, e;
    up.steps_of(lo, hi, a, e);
    s0 = count - e;
    s1 = count - a;
  }
};
template <class T>
__device__ __forceinline__ ReversedTiles<T> reversed(const T& t) {
  return ReversedTiles<T>{t, t.count};
}
// Dense tiles from the last one down, [t0, te) visited te-1, te-2, ...
struct DenseTilesDown {
  int te, count;
  __device__ __forceinline__ int tile(int m) const {
    return __builtin_amdgcn_readfirstlane(te - 1 - m);
  }
  __device__ __forceinline__ void steps_of(int lo, int hi, int& s0, int& s1) const {
    s0 = min(max(te - hi, 0), count);
    s1 = min(max(te - lo, s0), count);
  }
};
__device__ __forceinline__ DenseTilesDown reversed(const DenseTiles& t) {
  return DenseTilesDown{t.t0 + t.count, t.count};
}
// The listed blocks (already in LDS, ascending, n entries) trimmed to the
// tile range [tb, te).
template <int TPB>
__device__ __forceinline__ SparseTiles<TPB> sparse_tiles(const int* lst, int n, int tb, int te) {
  // a: first block not wholly before tb; e: first block wholly at or past te.
  int a = 0, hi = n;
  while (a < hi) {
    const int mid = (a + hi) >> 1;
    if (lst[mid] * TPB + TPB > tb) hi = mid; else a = mid + 1;
  }
  int e = a;
  hi = n;
  while (e < hi) {
    const int mid = (e + hi) >> 1;
    if (lst[mid] * TPB >= te) hi = mid; else e = mid + 1;
  }
  if (a >= e || te <= tb) return SparseTiles<TPB>{lst + a, 0, 0, 0};
  const int s = max(tb - lst[a] * TPB, 0);
  const int tail = max((lst[e - 1] + 1) * TPB - te, 0);
  return SparseTiles<TPB>{lst + a, e - a, s, (e - a) * TPB - s - tail};
}

// Calls f(causal_tag, sparse_tag) with the compile-time flags of the call's
// masks (host side, for the launchers).
template <typename F>
hipError_t dispatch_mask(const Params& p, F&& f) {
  if (p.blk != nullptr)
    return p.causal ? f(std::true_type{}, std::true_type{}) : f(std::false_type{}, std::true_type{});
  return p.causal ? f(std::true_type{}, std::false_type{}) : f(std::false_type{}, std::false_type{});
}
// The same with a third flag, set when the window has a lower edge: only
// then can masked tiles come before the unmasked ones in a query-outer
// sweep, and kernels without that case keep a shorter loop structure.
template <typename F>
hipError_t dispatch_mask_win(const Params& p, F&& f) {
  if (p.win_left >= 0)
    return dispatch_mask(p, [&](auto c, auto s) { return f(c, s, std::true_type{}); });
  return dispatch_mask(p, [&](auto c, auto s) { return f(c, s, std::false_type{}); });
}

}  // namespace fa
