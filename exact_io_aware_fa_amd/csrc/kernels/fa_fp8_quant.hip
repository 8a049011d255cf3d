// Blockwise E4M3 encoding of Q, K or V for the FP8 forward, for gfx950.
//
// Method: page 2 ("4. FlashAttention 深度剖析"), 4.5.4 (FP8 support): every
// block is scaled once and its scale kept; Q and K may first be rotated by a
// random Hadamard matrix. E4M3's range (largest magnitude 448, smallest
// normal 2^-6) is the page's exercise 3.
//
// A block is 128 rows of one head. Its scale is the power of two 2^e with e
// the smallest integer such that max |x| <= 448 * 2^e, so x * 2^-e is exact
// and the only rounding is the conversion to E4M3 (v_cvt_pk_fp8_f32: round to
// nearest even, with subnormals). With a rotation the block is x R, R =
// diag(signs) H_d (entries +-1, fast Walsh-Hadamard butterflies in fp32),
// and the stored scale is 2^e / sqrt(d), so scale * codes approximates
// x R / sqrt(d), the page's x H.
//
// Layouts written: rows -- codes [bh][np][d], as the attention kernel's Q
// and K operands want them; V -- codes [bh][nb][d][128], each block
// transposed (channel-major), so that the kernel's V^T operand reads are
// plain row reads. Rows past n are zero codes.
//
// One workgroup (256 threads) per block. The block's bf16 rows come from
// HBM straight into LDS with coalesced buffer loads (each wave load is 1 KB
// of consecutive bytes), the 16-byte chunks of row r XOR-swizzled so that
// the row reads below hit 16 different bank groups; rows past n read as
// zero through the buffer descriptor's size (and are zeroed on reading, as
// such lanes may leave LDS untouched). Thread t then holds half a row
// (row t / 2, channels (t % 2) * d/2 ...) in fp32 registers. The codes go
// back through LDS and leave with coalesced 16-byte stores (rows layout) or
// transposed (V layout).
#include "fa_device.h"

namespace fa {

namespace {

constexpr int kQThreads = 256;

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }

// Chunk swizzle of the staged block: a read phase (16 lanes) covers rows
// 0..7 (or 8..15, ...) at one logical chunk of each half row. (d = 256: a
// row is two full passes over the banks, so the two halves of a row share a
// bank group and the reads conflict two ways; this kernel is bound by HBM.)
template <int D>
__device__ __forceinline__ int qswz(int row) {
  return D >= 128 ? (row & 7) : ((row >> 1) & 3);
}

template <int D, bool ROT, bool VT>
__global__ __launch_bounds__(kQThreads) void fp8_quant_kernel(Fp8QuantParams p) {
  constexpr int HD = D / 2;        // channels per thread
  constexpr int CPR = D / 8;       // 16-byte bf16 chunks per row
  constexpr int LOADS = 128 * CPR / kQThreads;  // chunks per thread
  static_assert(HD % 16 == 0 && LOADS * kQThreads == 128 * CPR, "block split");
  __shared__ float red[kQThreads / 64];
  __shared__ __attribute__((aligned(1024))) bf16 xs[128 * D];
  // The codes reuse the staging buffer: every read of it precedes the block
  // maximum's barrier. (Half the LDS per workgroup, so more blocks per CU
  // hide the HBM latency.)
  uint8_t* const cs = reinterpret_cast<uint8_t*>(xs);

  const int blk = blockIdx.x;
  const int bh = blockIdx.y;
  const int t = threadIdx.x;
  const int w = t >> 6;
  const int lane = t & 63;
  const int r = t >> 1;
  const int hh = t & 1;

  // Stage the block: wave w's load i fills LDS chunks (w * LOADS + i) * 64 +
  // lane, i.e. row q / CPR, physical chunk q % CPR, which holds logical chunk
  // (q % CPR) ^ qswz(row).
  {
    const size_t row0 = (size_t)bh * p.n + (size_t)blk * 128;
    const int rows = max(min(p.n - blk * 128, 128), 0);
    const auto rs = buffer_rsrc(static_cast<const bf16*>(p.x) + row0 * D, rows * D * 2);
#pragma unroll
    for (int i = 0; i < LOADS; ++i) {
      const int q = (w * LOADS + i) * 64 + lane;
      const int row = q / CPR;
      const int voff = (row * CPR + ((q % CPR) ^ qswz<D>(row))) * 16;
      bload_lds16(rs, voff, xs + (w * LOADS + i) * 64 * 8);
    }
    wait_global_loads();
    __syncthreads();
  }

  // Rows past n: out-of-range lanes of a load into LDS may leave their
  // bytes as they were, so those rows are zeroed here, not read.
  const bool live = blk * 128 + r < p.n;
  float x[HD];
#pragma unroll
  for (int i = 0; i < HD / 8; ++i) {
    const int chunk = (hh * (HD / 8) + i) ^ qswz<D>(r);
    u32x4 v = ld16(xs + (r * CPR + chunk) * 8);
    if (!live) v = u32x4{0u, 0u, 0u, 0u};
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      x[8 * i + 2 * j] = bf16_lo(v[j]);
      x[8 * i + 2 * j + 1] = bf16_hi(v[j]);
    }
  }

  if (ROT) {
    // x <- x diag(signs) H_d. H_d is the product of one +-butterfly per
    // index bit; bits below log2(d/2) are inside the thread, the top bit
    // pairs the two halves of the row (lanes t and t ^ 1).
#pragma unroll
    for (int i = 0; i < HD / 16; ++i) {
      const u32x4 sv = ld16(p.signs + hh * HD + 16 * i);
#pragma unroll
      for (int j = 0; j < 16; ++j) {
        const int8_t sg = (int8_t)((sv[j >> 2] >> (8 * (j & 3))) & 0xFF);
        x[16 * i + j] = sg < 0 ? -x[16 * i + j] : x[16 * i + j];
      }
    }
#pragma unroll
    for (int h = 1; h < HD; h <<= 1)
#pragma unroll
      for (int i = 0; i < HD; ++i)
        if (!(i & h)) {
          const float a = x[i], b = x[i + h];
          x[i] = a + b;
          x[i + h] = a - b;
        }
#pragma unroll
    for (int i = 0; i < HD; ++i) {
      const float y = __shfl_xor(x[i], 1);
      x[i] = hh ? (y - x[i]) : (x[i] + y);
    }
  }

  // Block maximum of |x|.
  float am = 0.f;
#pragma unroll
  for (int i = 0; i < HD; ++i) am = fmaxf(am, fabsf(x[i]));
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) am = fmaxf(am, __shfl_xor(am, o));
  if (lane == 0) red[w] = am;
  __syncthreads();
  am = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));

  // Smallest e with am <= 448 * 2^e: am = m 2^E, m in [0.5, 1), and
  // 448 = 0.875 * 2^9.
  int E;
  const float m = frexpf(am, &E);
  const int e = am == 0.f ? 0 : (m <= 0.875f ? E - 9 : E - 8);
  if (t == 0) p.scales[(size_t)bh * p.nb + blk] = ldexpf(1.f, e) * p.post;

  // Codes into LDS, row-major [128][D] bytes, 16-byte chunks of a row
  // swizzled like the input (same conflict-free pattern, bytes instead of
  // bf16: a half row is HD / 16 chunks).
#pragma unroll
  for (int i = 0; i < HD / 16; ++i) {
    u32x4 o;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int k = 16 * i + 4 * q;
      uint32_t c = __builtin_amdgcn_cvt_pk_fp8_f32(ldexpf(x[k], -e), ldexpf(x[k + 1], -e), 0u,
                                                   false);
      c = __builtin_amdgcn_cvt_pk_fp8_f32(ldexpf(x[k + 2], -e), ldexpf(x[k + 3], -e), c, true);
      o[q] = c;
    }
    const int chunk = hh * (HD / 16) + i;
    *reinterpret_cast<u32x4*>(cs + r * D + ((chunk ^ (r & (D / 16 - 1))) << 4)) = o;
  }
  __syncthreads();

  if (!VT) {
    // Coalesced: thread t stores 16-byte chunks t, t + 256, ... of the block.
    uint8_t* dst = p.codes + ((size_t)bh * p.np + (size_t)blk * 128) * D;
    constexpr int CC = D / 16;  // code chunks per row
#pragma unroll
    for (int i = 0; i < 128 * CC / kQThreads; ++i) {
      const int q = i * kQThreads + t;
      const int row = q / CC, cc = q % CC;
      *reinterpret_cast<u32x4*>(dst + (size_t)q * 16) =
          ld16(cs + row * D + ((cc ^ (row & (CC - 1))) << 4));
    }
  } else {
    // Transposed block: output row c (channel) holds the block's 128 keys.
    constexpr int TPC = kQThreads / D;  // threads per output row
    constexpr int KPT = 128 / TPC;      // keys per thread
    const int c = t / TPC;
    const int k0 = (t % TPC) * KPT;
    const int cchunk = c >> 4;
    uint8_t* dst = p.codes + ((size_t)bh * p.nb + blk) * (size_t)(D * 128) + c * 128 + k0;
#pragma unroll
    for (int ch = 0; ch < KPT / 16; ++ch) {
      u32x4 o;
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        uint32_t v = 0;
#pragma unroll
        for (int b = 0; b < 4; ++b) {
          const int key = k0 + 16 * ch + 4 * q + b;
          const int phys = (cchunk ^ (key & (D / 16 - 1))) * 16 + (c & 15);
          v |= (uint32_t)cs[key * D + phys] << (8 * b);
        }
        o[q] = v;
      }
      *reinterpret_cast<u32x4*>(dst + 16 * ch) = o;
    }
  }
}

template <int D>
hipError_t launch_d(const Fp8QuantParams& p, hipStream_t s) {
  dim3 grid((unsigned)p.nb, (unsigned)p.bh), block(kQThreads);
  const bool rot = p.signs != nullptr;
  if (p.vt) {
    if (rot) return hipErrorInvalidValue;
    hipLaunchKernelGGL((fp8_quant_kernel<D, false, true>), grid, block, 0, s, p);
  } else if (rot) {
    hipLaunchKernelGGL((fp8_quant_kernel<D, true, false>), grid, block, 0, s, p);
  } else {
    hipLaunchKernelGGL((fp8_quant_kernel<D, false, false>), grid, block, 0, s, p);
  }
  return hipGetLastError();
}

}  // namespace

hipError_t launch_fp8_quantize(const Fp8QuantParams& p, int d, hipStream_t s) {
  switch (d) {
    case 64: return launch_d<64>(p, s);
    case 128: return launch_d<128>(p, s);
    case 256: return launch_d<256>(p, s);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace fa
