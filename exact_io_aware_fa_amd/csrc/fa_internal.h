// Internal interface between the C-ABI layer (fa_api.hip) and the kernel
// translation units. Not installed; not part of the ABI.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace fa {

// Everything a kernel needs about one call; passed by value as a kernel
// argument. Byte offsets inside one head's rows fit in 31 bits (enforced by
// validation); head bases are 64-bit.
//
// Batch entries and memory: entry b (a batch element, or one sequence of a
// packed variable-length batch) owns rows start .. start + len - 1 of each
// head. Without cu_seqlens, entry b is memory batch b with start = 0 and
// len = rows = n. With cu_seqlens, every entry lives in the single memory
// batch [heads, rows, d], start = cu_seqlens[b], len = its length (at most
// n, the longest), and rows = the packed total.
struct Params {
  const void* q;
  const void* k;
  const void* v;
  const void* o_in;     // backward: forward output
  const void* d_o;      // backward: upstream gradient
  const int32_t* kv_len;  // nullable, device int32[batch]
  const int32_t* cu_seqlens;  // nullable, device int32[batch + 1]: packed batch
  void* o;              // forward output
  float* lse;           // forward output / backward input, fp32, one per Q row
  void* dq;
  void* dk;
  void* dv;
  float* dvec;          // backward workspace: D_i = <dO_i, O_i>, [batch*H][n_pad]
  float* l2vec;         // backward workspace: L_i * log2(e), [batch*H][n_pad]
  float* dq_acc;        // fp32 dQ accumulator to zero (fp32 path: dq itself)
  int batch;
  int heads;            // query heads (Q, O, dO, dQ, LSE)
  int heads_kv;         // K/V heads (K, V, dK, dV); divides heads
  int group;            // heads / heads_kv: query heads per K/V head
  int n;                // sequence length (packed batch: the longest one)
  int rows;             // rows per head in memory (n, or the packed total)
  int n_pad;            // n rounded up to a multiple of 64 (workspace rows)
  int causal;
  int win_left;         // sliding window: keys j >= i - win_left (-1: unbounded)
  int win_right;        // sliding window: keys j <= i + win_right (-1: unbounded)
  const int32_t* blk;   // nullable: block-sparse index (see fa_device.h)
  int nb;               // blocks per side of the block mask
  // Scores enter exp2 as s * c where c = |scale| * log2(e), raised to at
  // least FLT_MIN so that c > 0 and hidden entries (-inf) stay -inf; a
  // negative scale is applied by negating Q (exact), flagged by q_neg.
  float c;
  float scale;          // signed softmax scale (backward gradient factor)
  int q_neg;
};

// FP8 (E4M3) forward. Codes of Q and K are [batch*heads][np][d] bytes, V's
// [batch*heads_kv][nb][d][128] (each 128-key block transposed); rows past n
// hold zero codes. One float scale per (head, 128-row block); V's scales
// are powers of two.
struct Fp8Params {
  const uint8_t* q8;
  const uint8_t* k8;
  const uint8_t* v8;
  const float* q_scale;   // [batch*heads][nb]
  const float* k_scale;   // [batch*heads_kv][nb]
  const float* v_scale;   // [batch*heads_kv][nb]
  const int32_t* kv_len;  // nullable, device int32[batch]
  void* o;                // bf16 [batch, heads, n, d]
  float* lse;             // [batch, heads, n]
  int batch;
  int heads;
  int heads_kv;
  int group;
  int n;
  int np;                 // n rounded up to a multiple of 128
  int nb;                 // np / 128
  int causal;
  float c;                // |scale| * log2(e), at least FLT_MIN
  int q_neg;              // negative scale: Q codes are negated (sign bit)
};

// Blockwise E4M3 encoding of one bf16 tensor [bh][n][d].
struct Fp8QuantParams {
  const void* x;          // bf16
  const int8_t* signs;    // nullable: rotate by diag(signs) H_d first
  uint8_t* codes;
  float* scales;
  int bh;                 // batch * heads
  int n;
  int np;
  int nb;
  int vt;                 // 1: V layout (blocks transposed), 0: rows
  float post;             // factor folded into the stored scales (1/sqrt(d) if rotated)
};

hipError_t launch_fp8_quantize(const Fp8QuantParams& p, int d, hipStream_t s);
hipError_t launch_fwd_fp8(const Fp8Params& p, int d, hipStream_t s);

hipError_t launch_fwd_bf16(const Params& p, int d, hipStream_t s);
hipError_t launch_fwd_bf16_d64(const Params& p, int d, hipStream_t s);
hipError_t launch_fwd_fp32(const Params& p, int d, hipStream_t s);
hipError_t launch_bwd_prep(const Params& p, int d, bool bf16, hipStream_t s);
hipError_t launch_bwd_dkdv_bf16(const Params& p, int d, hipStream_t s);
hipError_t launch_bwd_dkdv_bf16_d64(const Params& p, int d, hipStream_t s);
hipError_t launch_bwd_dkdv_bf16_d256(const Params& p, int d, hipStream_t s);
hipError_t launch_bwd_dkdv_bf16_wide(const Params& p, int d, hipStream_t s);
hipError_t launch_bwd_dq_bf16(const Params& p, int d, hipStream_t s);
hipError_t launch_bwd_dq_bf16_d256(const Params& p, int d, hipStream_t s);
hipError_t launch_bwd_fp32(const Params& p, int d, hipStream_t s);
hipError_t launch_block_index(const uint8_t* mask, int nb, int32_t* out, hipStream_t s);

}  // namespace fa
