// Block-sparse index: turns a block mask over kBlock x kBlock blocks (device
// uint8 [nb][nb], nonzero = the block is visible) into the per-row lists of
// visible key blocks and the per-column lists of query blocks, ascending,
// in the layout the attention kernels read (fa_device.h). Block-sparse
// attention with a coarse block-level mask whose empty blocks are skipped:
// page 3, "深入浅出 FlashAttention", 第八部分.
//
// One workgroup of 16 waves: a wave takes whole rows (then columns), counts
// their visible blocks 64 at a time with a ballot, a single lane turns the
// counts into offsets, and the waves write each list in order. nb <= 1024.
#include "fa_device.h"

namespace fa {

namespace {

constexpr int kThreads = 1024;

__global__ __launch_bounds__(kThreads) void block_index_kernel(const uint8_t* __restrict__ mask,
                                                               int nb, int32_t* __restrict__ out) {
  __shared__ int start[kMaxBlocks];
  const int lane = threadIdx.x & 63;
  const int w = threadIdx.x >> 6;
  constexpr int NW = kThreads / 64;
  int32_t* const row_ptr = out;
  int32_t* const col_idx = out + nb + 1;
  int32_t* const col_ptr = col_idx + nb * nb;
  int32_t* const row_idx = col_ptr + nb + 1;
  for (int pass = 0; pass < 2; ++pass) {
    // pass 0: row r lists the key blocks j with mask[r][j] set;
    // pass 1: column r lists the query blocks j with mask[j][r] set.
    int32_t* const ptr = pass == 0 ? row_ptr : col_ptr;
    int32_t* const idx = pass == 0 ? col_idx : row_idx;
    auto visible = [&](int r, int j) {
      if (j >= nb) return false;
      const size_t at = pass == 0 ? (size_t)r * nb + j : (size_t)j * nb + r;
      return mask[at] != 0;
    };
    for (int r = w; r < nb; r += NW) {
      int count = 0;
      for (int j0 = 0; j0 < nb; j0 += 64)
        count += __builtin_popcountll(__builtin_amdgcn_ballot_w64(visible(r, j0 + lane)));
      if (lane == 0) start[r] = count;
    }
    __syncthreads();
    if (threadIdx.x == 0) {
      int acc = 0;
      for (int r = 0; r < nb; ++r) {
        const int c = start[r];
        start[r] = acc;
        ptr[r] = acc;
        acc += c;
      }
      ptr[nb] = acc;
    }
    __syncthreads();
    for (int r = w; r < nb; r += NW) {
      int pos = start[r];
      for (int j0 = 0; j0 < nb; j0 += 64) {
        const bool v = visible(r, j0 + lane);
        const uint64_t bal = __builtin_amdgcn_ballot_w64(v);
        if (v) idx[pos + __builtin_popcountll(bal & ((uint64_t(1) << lane) - 1))] = j0 + lane;
        pos += __builtin_popcountll(bal);
      }
    }
    __syncthreads();
  }
}

}  // namespace

hipError_t launch_block_index(const uint8_t* mask, int nb, int32_t* out, hipStream_t s) {
  if (nb < 1 || nb > kMaxBlocks) return hipErrorInvalidValue;
  hipLaunchKernelGGL(block_index_kernel, dim3(1), dim3(kThreads), 0, s, mask, nb, out);
  return hipGetLastError();
}

}  // namespace fa
