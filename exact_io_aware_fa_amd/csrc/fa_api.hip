// C-ABI entry points (include/fa.h): argument validation, workspace layout,
// kernel dispatch. Host code only; the kernels live in kernels/*.hip.
//
// Validation runs on the host before anything is enqueued and touches no HIP
// state, so every error path is reachable without a GPU.
#include <float.h>
#include <math.h>
#include <stdint.h>

#include <mutex>

#include "../../include/fa.h"
#include "fa_internal.h"

// Scratch of fa_bwd_noalloc: the backward workspace (the D and L log2 e
// vectors) for callers that cannot allocate. One copy per device, at its own
// device address, held until the process ends. In host code `scratch` names
// a host-side stand-in, never the device memory: the device address comes
// from noalloc_scratch() below and is the only one ever passed to a kernel.
static __device__ __align__(256) unsigned char scratch[FA_NOALLOC_SCRATCH_BYTES];

namespace {

constexpr int64_t kMaxN = int64_t(1) << 22;

struct Range {
  uintptr_t lo, hi;  // [lo, hi)
};

Range range_of(const void* p, size_t bytes) {
  const uintptr_t a = reinterpret_cast<uintptr_t>(p);
  return Range{a, a + bytes};
}

bool overlaps(Range a, Range b) { return a.lo < b.hi && b.lo < a.hi; }

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

size_t elem_size(fa_dtype t) { return t == FA_BF16 ? 2 : 4; }

int64_t n_padded(int64_t n) { return (n + 63) / 64 * 64; }

// The shape of one call. A batch entry is a batch element (padded layout,
// [batch, heads, n, d]) or one sequence of a packed batch ([heads, total, d]
// with offsets cu_seqlens); see Params for how kernels address them.
struct Shape {
  int64_t entries;   // batch elements, or sequences of a packed batch
  int64_t heads;
  int64_t heads_kv;
  int64_t n;         // sequence length (packed: the longest sequence)
  int64_t rows;      // rows per head in memory (n, or the packed total)
  int64_t mem_batch; // leading dimension in memory (entries, or 1 if packed)
  int64_t d;
  const int32_t* cu_seqlens;  // packed batches only
};

Shape padded_shape(int64_t batch, int64_t heads, int64_t heads_kv, int64_t n, int64_t d) {
  return Shape{batch, heads, heads_kv, n, n, batch, d, nullptr};
}

Shape packed_shape(int64_t num_seqs, int64_t heads, int64_t heads_kv, int64_t total,
                   int64_t max_seqlen, int64_t d, const int32_t* cu_seqlens) {
  return Shape{num_seqs, heads, heads_kv, max_seqlen, total, 1, d, cu_seqlens};
}

fa_status check_shape(const Shape& s, float scale, fa_dtype dtype) {
  if (s.entries < 1 || s.heads < 1 || s.n < 1 || s.n > kMaxN) return FA_E_SHAPE;
  if (s.rows < s.n) return FA_E_SHAPE;  // a packed sequence fits in the total
  if (s.entries > INT32_MAX - 1 || s.heads > INT32_MAX || s.rows > INT32_MAX) return FA_E_SHAPE;
  // Grouped K/V heads: every K/V head serves the same number of query heads.
  if (s.heads_kv < 1 || s.heads_kv > s.heads || s.heads % s.heads_kv != 0) return FA_E_SHAPE;
  if (s.d != 64 && s.d != 128 && s.d != 256) return FA_E_UNSUPPORTED;
  if (dtype != FA_BF16 && dtype != FA_FP32) return FA_E_UNSUPPORTED;
  if (!isfinite(scale)) return FA_E_UNSUPPORTED;
  // Byte offsets inside one head's rows are 31-bit; workgroup counts must fit
  // a grid.
  if (s.rows * s.d * int64_t(elem_size(dtype)) >= (int64_t(1) << 31)) return FA_E_SHAPE;
  const int64_t tiles = (s.n + 63) / 64;
  if (tiles * s.entries * s.heads >= (int64_t(1) << 31)) return FA_E_SHAPE;
  return FA_OK;
}

// One per-entry-padded fp32 vector of the backward workspace (D or L log2 e).
size_t vec_bytes(int64_t entries, int64_t heads, int64_t n) {
  const size_t b = size_t(entries) * size_t(heads) * size_t(n_padded(n)) * sizeof(float);
  return (b + 255) & ~size_t(255);
}

// Bytes of a tensor with `nh` heads, and of the LSE.
size_t tensor_bytes(const Shape& s, int64_t nh, fa_dtype dtype) {
  return size_t(s.mem_batch) * size_t(nh) * size_t(s.rows) * size_t(s.d) * elem_size(dtype);
}
size_t lse_bytes(const Shape& s) {
  return size_t(s.mem_batch) * size_t(s.heads) * size_t(s.rows) * sizeof(float);
}

int64_t mask_blocks(int64_t n) { return (n + 127) / 128; }

size_t block_index_bytes(int64_t n) {
  const int64_t nb = mask_blocks(n);
  return size_t(2 * (nb + 1) + 2 * nb * nb) * sizeof(int32_t);
}

fa::Params base_params(const Shape& s, int causal, float scale) {
  fa::Params p{};
  p.win_left = -1;
  p.win_right = -1;
  p.cu_seqlens = s.cu_seqlens;
  p.batch = int(s.entries);
  p.heads = int(s.heads);
  p.heads_kv = int(s.heads_kv);
  p.group = int(s.heads / s.heads_kv);
  p.n = int(s.n);
  p.rows = int(s.rows);
  p.n_pad = int(n_padded(s.n));
  p.causal = causal ? 1 : 0;
  float c = fabsf(scale) * 1.4426950408889634f;
  p.c = c < FLT_MIN ? FLT_MIN : c;
  p.scale = scale;
  p.q_neg = scale < 0.f ? 1 : 0;
  return p;
}

// Checks the optional masks and records them in p. Window sides beyond the
// sequence length act as unbounded, so they are stored clamped to n.
fa_status check_mask(const Shape& sh, const fa_mask* mask, fa::Params& p) {
  if (mask == nullptr) return FA_OK;
  if (mask->window_left < -1 || mask->window_right < -1) return FA_E_SHAPE;
  p.win_left = int(mask->window_left < sh.n ? mask->window_left : sh.n);
  p.win_right = int(mask->window_right < sh.n ? mask->window_right : sh.n);
  if (mask->block_index != nullptr) {
    if (mask_blocks(sh.n) > 1024) return FA_E_UNSUPPORTED;
    if (reinterpret_cast<uintptr_t>(mask->block_index) & 3u) return FA_E_ALIGN;
    p.blk = mask->block_index;
    p.nb = int(mask_blocks(sh.n));
  }
  return FA_OK;
}

Range index_range(const Shape& sh, const fa_mask* mask) {
  if (mask == nullptr || mask->block_index == nullptr) return Range{0, 0};
  return range_of(mask->block_index, block_index_bytes(sh.n));
}

// The small device array an entry point reads besides the tensors: the key
// lengths (padded batches) or the sequence offsets (packed batches).
Range aux_range(const Shape& sh, const int32_t* kv_len) {
  if (kv_len) return range_of(kv_len, size_t(sh.entries) * sizeof(int32_t));
  if (sh.cu_seqlens) return range_of(sh.cu_seqlens, size_t(sh.entries + 1) * sizeof(int32_t));
  return Range{0, 0};
}

fa_status fwd_impl(const Shape& sh, int causal, float softmax_scale, fa_dtype dtype,
                   const void* q, const void* k, const void* v, const int32_t* kv_len,
                   const fa_mask* mask, void* o, float* lse, void* stream) {
  fa_status st = check_shape(sh, softmax_scale, dtype);
  if (st != FA_OK) return st;
  fa::Params p = base_params(sh, causal, softmax_scale);
  st = check_mask(sh, mask, p);
  if (st != FA_OK) return st;
  if (!q || !k || !v || !o || !lse) return FA_E_NULLPTR;
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(o) || !aligned16(lse))
    return FA_E_ALIGN;
  const Range ra = aux_range(sh, kv_len);
  if (ra.lo & 3u) return FA_E_ALIGN;
  const size_t tb = tensor_bytes(sh, sh.heads, dtype);
  const size_t kb = tensor_bytes(sh, sh.heads_kv, dtype);
  const Range ins[3] = {range_of(q, tb), range_of(k, kb), range_of(v, kb)};
  const Range ro = range_of(o, tb), rl = range_of(lse, lse_bytes(sh));
  if (overlaps(ro, rl)) return FA_E_ALIAS;
  for (const Range& r : ins)
    if (overlaps(r, ro) || overlaps(r, rl)) return FA_E_ALIAS;
  if (overlaps(ra, ro) || overlaps(ra, rl)) return FA_E_ALIAS;
  const Range ri = index_range(sh, mask);
  if (overlaps(ri, ro) || overlaps(ri, rl)) return FA_E_ALIAS;

  p.q = q;
  p.k = k;
  p.v = v;
  p.kv_len = kv_len;
  p.o = o;
  p.lse = lse;
  hipStream_t s = static_cast<hipStream_t>(stream);
  const hipError_t e = (dtype == FA_BF16) ? fa::launch_fwd_bf16(p, int(sh.d), s)
                                          : fa::launch_fwd_fp32(p, int(sh.d), s);
  return e == hipSuccess ? FA_OK : FA_E_LAUNCH;
}

fa_status bwd_impl(const Shape& sh, int causal, float softmax_scale, fa_dtype dtype,
                   const void* q, const void* k, const void* v, const void* o,
                   const void* d_o, const float* lse, const int32_t* kv_len,
                   const fa_mask* mask, void* dq, void* dk, void* dv, void* workspace,
                   size_t workspace_bytes, void* stream, void* const events[4]) {
  fa_status st = check_shape(sh, softmax_scale, dtype);
  if (st != FA_OK) return st;
  fa::Params p = base_params(sh, causal, softmax_scale);
  st = check_mask(sh, mask, p);
  if (st != FA_OK) return st;
  if (!q || !k || !v || !o || !d_o || !lse || !dq || !dk || !dv) return FA_E_NULLPTR;
  if (!workspace) return FA_E_WORKSPACE;
  const size_t need = 2 * vec_bytes(sh.entries, sh.heads, sh.n);
  if (workspace_bytes < need) return FA_E_WORKSPACE;
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(o) || !aligned16(d_o) ||
      !aligned16(lse) || !aligned16(dq) || !aligned16(dk) || !aligned16(dv))
    return FA_E_ALIGN;
  if ((reinterpret_cast<uintptr_t>(workspace) & 255u) != 0) return FA_E_ALIGN;
  const Range ra = aux_range(sh, kv_len);
  if (ra.lo & 3u) return FA_E_ALIGN;

  const size_t tb = tensor_bytes(sh, sh.heads, dtype);
  const size_t kb = tensor_bytes(sh, sh.heads_kv, dtype);
  const Range ins[8] = {range_of(q, tb), range_of(k, kb),  range_of(v, kb),
                        range_of(o, tb), range_of(d_o, tb), range_of(lse, lse_bytes(sh)),
                        ra,              index_range(sh, mask)};
  const Range outs[4] = {range_of(dq, tb), range_of(dk, kb), range_of(dv, kb),
                         range_of(workspace, need)};
  for (int i = 0; i < 4; ++i) {
    for (int j = 0; j < 8; ++j)
      if (overlaps(outs[i], ins[j])) return FA_E_ALIAS;
    for (int j = i + 1; j < 4; ++j)
      if (overlaps(outs[i], outs[j])) return FA_E_ALIAS;
  }

  p.q = q;
  p.k = k;
  p.v = v;
  p.o_in = o;
  p.d_o = d_o;
  p.lse = const_cast<float*>(lse);
  p.kv_len = kv_len;
  p.dq = dq;
  p.dk = dk;
  p.dv = dv;
  p.dvec = static_cast<float*>(workspace);
  p.l2vec = reinterpret_cast<float*>(static_cast<char*>(workspace) +
                                     vec_bytes(sh.entries, sh.heads, sh.n));
  // fp32: the backward adds dQ into the caller's dq with atomics, after the
  // prep kernel has zeroed the rows it covers.
  p.dq_acc = (dtype == FA_FP32) ? static_cast<float*>(dq) : nullptr;
  hipStream_t s = static_cast<hipStream_t>(stream);
  auto mark = [&](int i) -> hipError_t {
    if (events == nullptr || events[i] == nullptr) return hipSuccess;
    return hipEventRecord(static_cast<hipEvent_t>(events[i]), s);
  };
  const int d = int(sh.d);
  hipError_t e = mark(0);
  if (dtype == FA_BF16) {
    // bf16: the query-outer dQ kernel also forms D_i and L_i log2(e) for its
    // rows and writes them to the workspace, so it runs first and the dK/dV
    // kernel, which reads them, second (two launches).
    if (e == hipSuccess) e = fa::launch_bwd_dq_bf16(p, d, s);
    if (e == hipSuccess) e = mark(1);
    if (e == hipSuccess) e = fa::launch_bwd_dkdv_bf16(p, d, s);
  } else {
    // fp32: D_i, L_i log2(e) and the zeroed dQ accumulator come from the
    // prep kernel, then one kernel adds dQ with atomics and writes dK, dV.
    if (e == hipSuccess) e = fa::launch_bwd_prep(p, d, false, s);
    if (e == hipSuccess) e = mark(1);
    if (e == hipSuccess) e = fa::launch_bwd_fp32(p, d, s);
  }
  if (e == hipSuccess) e = mark(2);
  if (e == hipSuccess) e = mark(3);
  return e == hipSuccess ? FA_OK : FA_E_LAUNCH;
}

// FP8 encoded tensors: np rows per head (n rounded up to a block), one
// scale per block.
int64_t fp8_rows(int64_t n) { return (n + 127) / 128 * 128; }
size_t fp8_codes_bytes(int64_t bh, int64_t n, int64_t d) { return size_t(bh * fp8_rows(n) * d); }
size_t fp8_scales_bytes(int64_t bh, int64_t n) { return size_t(bh * (fp8_rows(n) / 128)) * 4; }

fa_status check_fp8_shape(int64_t batch, int64_t heads, int64_t heads_kv, int64_t n) {
  if (batch < 1 || heads < 1 || n < 1 || n > kMaxN) return FA_E_SHAPE;
  if (batch > INT32_MAX - 1 || heads > INT32_MAX) return FA_E_SHAPE;
  if (heads_kv < 1 || heads_kv > heads || heads % heads_kv != 0) return FA_E_SHAPE;
  if (batch * heads * ((n + 127) / 128) >= (int64_t(1) << 31)) return FA_E_SHAPE;
  return FA_OK;
}

bool aligned4(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 3u) == 0; }

// Per-device address of `scratch`, looked up once per device with that device
// current (hipGetSymbolAddress), under a lock.
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch[kMaxDevices];

hipError_t noalloc_scratch(hipStream_t stream, void** out) {
  int dev = 0;
  hipError_t e = hipStreamGetDevice(stream, &dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> guard(g_scratch_mu);
  if (g_scratch[dev] == nullptr) {
    int cur = 0;
    e = hipGetDevice(&cur);
    if (e != hipSuccess) return e;
    if (cur != dev && (e = hipSetDevice(dev)) != hipSuccess) return e;
    void* ptr = nullptr;
    e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    if (cur != dev) {
      const hipError_t r = hipSetDevice(cur);
      if (e == hipSuccess) e = r;
    }
    if (e != hipSuccess) return e;
    if (ptr == nullptr || (reinterpret_cast<uintptr_t>(ptr) & 255u) != 0)
      return hipErrorInvalidSymbol;
    g_scratch[dev] = ptr;
  }
  *out = g_scratch[dev];
  return hipSuccess;
}

}  // namespace

extern "C" {

int fa_abi_version(void) { return FA_ABI_VERSION; }

size_t fa_fp8_codes_bytes(int64_t batch, int64_t heads, int64_t n, int64_t d) {
  if (check_fp8_shape(batch, heads, heads, n) != FA_OK || d < 1 || d > 256) return 0;
  return fp8_codes_bytes(batch * heads, n, d);
}

size_t fa_fp8_scales_bytes(int64_t batch, int64_t heads, int64_t n) {
  if (check_fp8_shape(batch, heads, heads, n) != FA_OK) return 0;
  return fp8_scales_bytes(batch * heads, n);
}

fa_status fa_fp8_quantize(int64_t batch, int64_t heads, int64_t n, int64_t d, int layout,
                          const void* x, const int8_t* signs, uint8_t* codes, float* scales,
                          void* stream) {
  fa_status st = check_fp8_shape(batch, heads, heads, n);
  if (st != FA_OK) return st;
  if (d != 64 && d != 128 && d != 256) return FA_E_UNSUPPORTED;
  if (layout != FA_FP8_ROWS && layout != FA_FP8_VT) return FA_E_UNSUPPORTED;
  if (layout == FA_FP8_VT && signs != nullptr) return FA_E_UNSUPPORTED;
  if (n * d * 2 >= (int64_t(1) << 31)) return FA_E_SHAPE;
  if (!x || !codes || !scales) return FA_E_NULLPTR;
  if (!aligned16(x) || !aligned16(codes) || !aligned4(scales)) return FA_E_ALIGN;
  if (signs && !aligned16(signs)) return FA_E_ALIGN;
  const int64_t bh = batch * heads;
  const Range rx = range_of(x, size_t(bh * n * d) * 2);
  const Range rs = signs ? range_of(signs, size_t(d)) : Range{0, 0};
  const Range rc = range_of(codes, fp8_codes_bytes(bh, n, d));
  const Range rk = range_of(scales, fp8_scales_bytes(bh, n));
  if (overlaps(rc, rk) || overlaps(rc, rx) || overlaps(rc, rs) || overlaps(rk, rx) ||
      overlaps(rk, rs))
    return FA_E_ALIAS;
  fa::Fp8QuantParams p{};
  p.x = x;
  p.signs = signs;
  p.codes = codes;
  p.scales = scales;
  p.bh = int(bh);
  p.n = int(n);
  p.np = int(fp8_rows(n));
  p.nb = p.np / 128;
  p.vt = layout == FA_FP8_VT ? 1 : 0;
  p.post = signs ? float(1.0 / sqrt(double(d))) : 1.f;
  const hipError_t e = fa::launch_fp8_quantize(p, int(d), static_cast<hipStream_t>(stream));
  return e == hipSuccess ? FA_OK : FA_E_LAUNCH;
}

fa_status fa_fwd_fp8(int64_t batch, int64_t heads, int64_t heads_kv, int64_t n, int64_t d,
                     int causal, float softmax_scale, const uint8_t* q8, const float* q_scales,
                     const uint8_t* k8, const float* k_scales, const uint8_t* v8,
                     const float* v_scales, const int32_t* kv_len, void* o, float* lse,
                     void* stream) {
  fa_status st = check_fp8_shape(batch, heads, heads_kv, n);
  if (st != FA_OK) return st;
  if (d != 64 && d != 128 && d != 256) return FA_E_UNSUPPORTED;
  if (!isfinite(softmax_scale)) return FA_E_UNSUPPORTED;
  if (n * d * 2 >= (int64_t(1) << 31)) return FA_E_SHAPE;
  if (!q8 || !q_scales || !k8 || !k_scales || !v8 || !v_scales || !o || !lse)
    return FA_E_NULLPTR;
  if (!aligned16(q8) || !aligned16(k8) || !aligned16(v8) || !aligned16(o)) return FA_E_ALIGN;
  if (!aligned4(q_scales) || !aligned4(k_scales) || !aligned4(v_scales) || !aligned4(lse) ||
      !aligned4(kv_len))
    return FA_E_ALIGN;
  const int64_t bq = batch * heads, bk = batch * heads_kv;
  const Range ins[7] = {range_of(q8, fp8_codes_bytes(bq, n, d)),
                        range_of(k8, fp8_codes_bytes(bk, n, d)),
                        range_of(v8, fp8_codes_bytes(bk, n, d)),
                        range_of(q_scales, fp8_scales_bytes(bq, n)),
                        range_of(k_scales, fp8_scales_bytes(bk, n)),
                        range_of(v_scales, fp8_scales_bytes(bk, n)),
                        kv_len ? range_of(kv_len, size_t(batch) * 4) : Range{0, 0}};
  const Range ro = range_of(o, size_t(bq * n * d) * 2);
  const Range rl = range_of(lse, size_t(bq * n) * 4);
  if (overlaps(ro, rl)) return FA_E_ALIAS;
  for (const Range& r : ins)
    if (overlaps(r, ro) || overlaps(r, rl)) return FA_E_ALIAS;
  fa::Fp8Params p{};
  p.q8 = q8;
  p.k8 = k8;
  p.v8 = v8;
  p.q_scale = q_scales;
  p.k_scale = k_scales;
  p.v_scale = v_scales;
  p.kv_len = kv_len;
  p.o = o;
  p.lse = lse;
  p.batch = int(batch);
  p.heads = int(heads);
  p.heads_kv = int(heads_kv);
  p.group = int(heads / heads_kv);
  p.n = int(n);
  p.np = int(fp8_rows(n));
  p.nb = p.np / 128;
  p.causal = causal ? 1 : 0;
  const float c = fabsf(softmax_scale) * 1.4426950408889634f;
  p.c = c < FLT_MIN ? FLT_MIN : c;
  p.q_neg = softmax_scale < 0.f ? 1 : 0;
  const hipError_t e = fa::launch_fwd_fp8(p, int(d), static_cast<hipStream_t>(stream));
  return e == hipSuccess ? FA_OK : FA_E_LAUNCH;
}

const char* fa_status_str(fa_status s) {
  switch (s) {
    case FA_OK: return "FA_OK";
    case FA_E_NULLPTR: return "FA_E_NULLPTR: a required pointer is NULL";
    case FA_E_SHAPE: return "FA_E_SHAPE: batch, heads, heads_kv, n or total out of range";
    case FA_E_UNSUPPORTED: return "FA_E_UNSUPPORTED: unsupported d, dtype or scale";
    case FA_E_WORKSPACE: return "FA_E_WORKSPACE: workspace missing or too small";
    case FA_E_ALIAS: return "FA_E_ALIAS: an output overlaps an input or another output";
    case FA_E_LAUNCH: return "FA_E_LAUNCH: kernel launch failed";
    case FA_E_ALIGN: return "FA_E_ALIGN: pointer not 16-byte aligned";
    case FA_E_SCRATCH:
      return "FA_E_SCRATCH: the call needs more scratch than fa_bwd_noalloc's static "
             "FA_NOALLOC_SCRATCH_BYTES buffer; use fa_bwd_gqa with a workspace";
  }
  return "FA_E_UNKNOWN";
}

size_t fa_bwd_workspace_bytes(int64_t batch, int64_t heads, int64_t n, int64_t d,
                              fa_dtype dtype) {
  // One padded slice per (batch entry, query head); a packed batch passes its
  // sequence count and longest length.
  if (check_shape(padded_shape(batch, heads, 1, n, d), 1.f, dtype) != FA_OK) return 0;
  return 2 * vec_bytes(batch, heads, n);
}

fa_status fa_fwd(int64_t batch, int64_t heads, int64_t n, int64_t d, int causal,
                 float softmax_scale, fa_dtype dtype, const void* q, const void* k,
                 const void* v, const int32_t* kv_len, void* o, float* lse,
                 void* stream) {
  return fwd_impl(padded_shape(batch, heads, heads, n, d), causal, softmax_scale, dtype, q, k,
                  v, kv_len, nullptr, o, lse, stream);
}

fa_status fa_fwd_gqa(int64_t batch, int64_t heads, int64_t heads_kv, int64_t n, int64_t d,
                     int causal, float softmax_scale, fa_dtype dtype, const void* q,
                     const void* k, const void* v, const int32_t* kv_len, void* o,
                     float* lse, void* stream) {
  return fwd_impl(padded_shape(batch, heads, heads_kv, n, d), causal, softmax_scale, dtype, q,
                  k, v, kv_len, nullptr, o, lse, stream);
}

fa_status fa_fwd_masked(int64_t batch, int64_t heads, int64_t heads_kv, int64_t n, int64_t d,
                        int causal, float softmax_scale, fa_dtype dtype, const void* q,
                        const void* k, const void* v, const int32_t* kv_len,
                        const fa_mask* mask, void* o, float* lse, void* stream) {
  return fwd_impl(padded_shape(batch, heads, heads_kv, n, d), causal, softmax_scale, dtype, q,
                  k, v, kv_len, mask, o, lse, stream);
}

fa_status fa_fwd_varlen(int64_t num_seqs, int64_t heads, int64_t heads_kv, int64_t total,
                        int64_t max_seqlen, int64_t d, const int32_t* cu_seqlens, int causal,
                        float softmax_scale, fa_dtype dtype, const void* q, const void* k,
                        const void* v, const fa_mask* mask, void* o, float* lse,
                        void* stream) {
  if (!cu_seqlens) return FA_E_NULLPTR;
  return fwd_impl(packed_shape(num_seqs, heads, heads_kv, total, max_seqlen, d, cu_seqlens),
                  causal, softmax_scale, dtype, q, k, v, nullptr, mask, o, lse, stream);
}

fa_status fa_bwd(int64_t batch, int64_t heads, int64_t n, int64_t d, int causal,
                 float softmax_scale, fa_dtype dtype, const void* q, const void* k,
                 const void* v, const void* o, const void* d_o, const float* lse,
                 const int32_t* kv_len, void* dq, void* dk, void* dv, void* workspace,
                 size_t workspace_bytes, void* stream) {
  return bwd_impl(padded_shape(batch, heads, heads, n, d), causal, softmax_scale, dtype, q, k,
                  v, o, d_o, lse, kv_len, nullptr, dq, dk, dv, workspace, workspace_bytes,
                  stream, nullptr);
}

fa_status fa_bwd_gqa(int64_t batch, int64_t heads, int64_t heads_kv, int64_t n, int64_t d,
                     int causal, float softmax_scale, fa_dtype dtype, const void* q,
                     const void* k, const void* v, const void* o, const void* d_o,
                     const float* lse, const int32_t* kv_len, void* dq, void* dk, void* dv,
                     void* workspace, size_t workspace_bytes, void* stream) {
  return bwd_impl(padded_shape(batch, heads, heads_kv, n, d), causal, softmax_scale, dtype, q,
                  k, v, o, d_o, lse, kv_len, nullptr, dq, dk, dv, workspace, workspace_bytes,
                  stream, nullptr);
}

fa_status fa_bwd_masked(int64_t batch, int64_t heads, int64_t heads_kv, int64_t n, int64_t d,
                        int causal, float softmax_scale, fa_dtype dtype, const void* q,
                        const void* k, const void* v, const void* o, const void* d_o,
                        const float* lse, const int32_t* kv_len, const fa_mask* mask, void* dq,
                        void* dk, void* dv, void* workspace, size_t workspace_bytes,
                        void* stream) {
  return bwd_impl(padded_shape(batch, heads, heads_kv, n, d), causal, softmax_scale, dtype, q,
                  k, v, o, d_o, lse, kv_len, mask, dq, dk, dv, workspace, workspace_bytes,
                  stream, nullptr);
}

fa_status fa_bwd_varlen(int64_t num_seqs, int64_t heads, int64_t heads_kv, int64_t total,
                        int64_t max_seqlen, int64_t d, const int32_t* cu_seqlens, int causal,
                        float softmax_scale, fa_dtype dtype, const void* q, const void* k,
                        const void* v, const void* o, const void* d_o, const float* lse,
                        const fa_mask* mask, void* dq, void* dk, void* dv, void* workspace,
                        size_t workspace_bytes, void* stream) {
  if (!cu_seqlens) return FA_E_NULLPTR;
  return bwd_impl(packed_shape(num_seqs, heads, heads_kv, total, max_seqlen, d, cu_seqlens),
                  causal, softmax_scale, dtype, q, k, v, o, d_o, lse, nullptr, mask, dq, dk,
                  dv, workspace, workspace_bytes, stream, nullptr);
}

fa_status fa_bwd_timed(int64_t batch, int64_t heads, int64_t heads_kv, int64_t n, int64_t d,
                       int causal, float softmax_scale, fa_dtype dtype, const void* q,
                       const void* k, const void* v, const void* o, const void* d_o,
                       const float* lse, const int32_t* kv_len, void* dq, void* dk, void* dv,
                       void* workspace, size_t workspace_bytes, void* stream,
                       void* const events[4]) {
  return bwd_impl(padded_shape(batch, heads, heads_kv, n, d), causal, softmax_scale, dtype, q,
                  k, v, o, d_o, lse, kv_len, nullptr, dq, dk, dv, workspace, workspace_bytes,
                  stream, events);
}

fa_status fa_bwd_noalloc(int64_t batch, int64_t heads, int64_t heads_kv, int64_t n, int64_t d,
                         int causal, float softmax_scale, fa_dtype dtype, const void* q,
                         const void* k, const void* v, const void* o, const void* d_o,
                         const float* lse, const int32_t* kv_len, void* dq, void* dk,
                         void* dv, void* stream) {
  // Sizes first, on the host only, so that a call too large for the static
  // buffer is rejected before any HIP call.
  const Shape sh = padded_shape(batch, heads, heads_kv, n, d);
  fa_status st = check_shape(sh, softmax_scale, dtype);
  if (st != FA_OK) return st;
  const size_t need = 2 * vec_bytes(sh.entries, sh.heads, sh.n);
  if (need > FA_NOALLOC_SCRATCH_BYTES) return FA_E_SCRATCH;
  void* ws = nullptr;
  if (noalloc_scratch(static_cast<hipStream_t>(stream), &ws) != hipSuccess) return FA_E_LAUNCH;
  // The backward's prep kernel writes every element of the workspace the
  // other kernels read, so nothing left by an earlier call is ever used.
  return bwd_impl(sh, causal, softmax_scale, dtype, q, k, v, o, d_o, lse, kv_len, nullptr, dq,
                  dk, dv, ws, FA_NOALLOC_SCRATCH_BYTES, stream, nullptr);
}

size_t fa_block_index_bytes(int64_t n) {
  if (n < 1 || mask_blocks(n) > 1024) return 0;
  return block_index_bytes(n);
}

fa_status fa_block_index_build(int64_t n, const uint8_t* block_mask, int32_t* index,
                               void* stream) {
  if (n < 1 || n > kMaxN) return FA_E_SHAPE;
  if (mask_blocks(n) > 1024) return FA_E_UNSUPPORTED;
  if (!block_mask || !index) return FA_E_NULLPTR;
  if (reinterpret_cast<uintptr_t>(index) & 3u) return FA_E_ALIGN;
  const int64_t nb = mask_blocks(n);
  if (overlaps(range_of(block_mask, size_t(nb * nb)), range_of(index, block_index_bytes(n))))
    return FA_E_ALIAS;
  const hipError_t e =
      fa::launch_block_index(block_mask, int(nb), index, static_cast<hipStream_t>(stream));
  return e == hipSuccess ? FA_OK : FA_E_LAUNCH;
}

}  // extern "C"
