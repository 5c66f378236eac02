// Per-tensor amax (two-stage) and the current-scaling FP8 cast for gfx950.
//
// Method: "Transformer Engine On ROCm and AMDGPU", "Two-stage amax Kernel":
// per-workgroup maxima, then one small reduction over them, no atomics.
// "Workflow: NVIDIA TransformerEngine FP8 Training Quickstart", Step 4:
// Float8CurrentScaling takes the scale from the current tensor; margin 0 as
// in the "Getting Started" (TE JAX) recipes.  Readings where the pages are
// silent: scale = fl32(fmt_max / amax) (1 when amax is 0, the largest finite
// float when the quotient overflows), scale_inv = fl32(1 / scale), and each
// element is the saturating round-to-nearest-even encode of fl32(x * scale).
//
// The maximum is taken over the |x| bit patterns as integers (exact for
// non-NaN bf16), so it does not depend on the reduction order.
#include <float.h>

#include <atomic>
#include <mutex>

#include "temx_device.h"

namespace temx {
namespace {

constexpr int kAmaxThreads = 256;
constexpr int kAmaxUnroll = 4;
constexpr int64_t kAmaxMaxBlocks = 1024;

int64_t amax_blocks(int64_t n) {
  const int64_t chunks = n / 8;
  int64_t b = (chunks + kAmaxThreads * kAmaxUnroll - 1) / (kAmaxThreads * kAmaxUnroll);
  if (b < 1) b = 1;
  return b > kAmaxMaxBlocks ? kAmaxMaxBlocks : b;
}

// The current-scaling cast's amax pass uses at most 512 workgroups: every cast
// workgroup reduces all partial maxima again, and fewer partials cost less
// there (measured on MI355X, 4096 x 4096 bf16: the whole cast 12.0-12.8 us
// with 512, 12.6-13.5 with 1024; 256 is slower on 8192 x 8192).
constexpr int64_t kCastAmaxBlocks = 512;

int64_t cast_amax_blocks(int64_t n) {
  const int64_t b = amax_blocks(n);
  return b > kCastAmaxBlocks ? kCastAmaxBlocks : b;
}

__device__ __forceinline__ uint32_t wave_max(uint32_t v) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) v = max(v, (uint32_t)__shfl_xor((int)v, off, 64));
  return v;
}

__device__ __forceinline__ uint32_t block_max(uint32_t v) {
  __shared__ uint32_t red[kAmaxThreads / 64];
  v = wave_max(v);
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = v;
  __syncthreads();
  uint32_t m = red[0];
#pragma unroll
  for (int i = 1; i < kAmaxThreads / 64; ++i) m = max(m, red[i]);
  return m;
}

// Stage one: grid-stride over 16-byte chunks; the n % 8 tail is read by
// block 0.  partial[blockIdx.x] = max |x| bits over the block's share.
// NT: non-temporal loads, for a standalone amax.  The current-scaling cast
// reads x again right after this pass and uses plain loads here, so that x is
// still in the last-level cache for its second read (measured on MI355X,
// 4096 x 4096 bf16: the whole cast 15.4 -> 12.9 us; the standalone amax is
// ~7% faster with non-temporal loads on 8192 x 8192).
template <bool NT>
__global__ __launch_bounds__(kAmaxThreads) void amax_partial_kernel(const uint16_t* __restrict__ x, int64_t n,
                                                                    uint32_t* __restrict__ partial) {
  const int64_t nchunks = n / 8;
  const uint4* xv = reinterpret_cast<const uint4*>(x);
  uint32_t m = 0;
  const int64_t stride = (int64_t)gridDim.x * kAmaxThreads * kAmaxUnroll;
  for (int64_t c0 = (int64_t)blockIdx.x * kAmaxThreads * kAmaxUnroll + threadIdx.x; c0 < nchunks; c0 += stride) {
    uint4 v[kAmaxUnroll];
#pragma unroll
    for (int u = 0; u < kAmaxUnroll; ++u) {
      const int64_t c = c0 + (int64_t)u * kAmaxThreads;
      v[u] = c < nchunks ? (NT ? load_nt16(xv + c) : xv[c]) : make_uint4(0, 0, 0, 0);
    }
#pragma unroll
    for (int u = 0; u < kAmaxUnroll; ++u) m = max(m, absmax_bits8(v[u]));
  }
  if (blockIdx.x == 0) {
    const int64_t i = nchunks * 8 + threadIdx.x;
    if (i < n) m = max(m, (uint32_t)(x[i] & 0x7FFFu));
  }
  m = block_max(m);
  if (threadIdx.x == 0) partial[blockIdx.x] = m;
}

// scale = fl32(fmt_max / amax) (1 for amax 0, the largest finite float when
// the quotient overflows).  A float32 quotient rounded once to float64 and
// then to float32 equals the correctly rounded float32 quotient (53 >=
// 2*24 + 2; Figueroa, "When is double rounding innocuous?", 1995), so this
// and 1 / scale below are IEEE float32 divisions.
template <int FMT>
__device__ __forceinline__ float current_scale(float amax) {
  float scale = 1.0f;
  if (amax != 0.0f) {
    scale = (float)((double)FmtTraits<FMT>::max_value / (double)amax);
    if (!(scale <= FLT_MAX)) scale = FLT_MAX;
  }
  return scale;
}

// Stage two of the standalone amax: one workgroup reduces the partial
// maxima.  (The current-scaling cast does this reduction inside its own
// workgroups, below.)
__global__ __launch_bounds__(kAmaxThreads) void amax_final_kernel(const uint32_t* __restrict__ partial, int nparts,
                                                                  float* __restrict__ amax_out) {
  uint32_t m = 0;
  for (int i = threadIdx.x; i < nparts; i += kAmaxThreads) m = max(m, partial[i]);
  m = block_max(m);
  if (threadIdx.x == 0) *amax_out = bf16_bits_to_float(m);
}

// Cast: y = fl32(x * scale), clamped to the finite range, then the plain
// round-to-nearest-even converts v_cvt_pk_{fp8,bf8}_f32.
template <int FMT>
__device__ __forceinline__ uint32_t cast4(uint32_t p0, uint32_t p1, float scale) {
  constexpr float mx = FmtTraits<FMT>::max_value;
  float a = __uint_as_float(p0 << 16) * scale, b = __uint_as_float(p0 & 0xFFFF0000u) * scale;
  float c = __uint_as_float(p1 << 16) * scale, d = __uint_as_float(p1 & 0xFFFF0000u) * scale;
  a = __builtin_amdgcn_fmed3f(a, -mx, mx);
  b = __builtin_amdgcn_fmed3f(b, -mx, mx);
  c = __builtin_amdgcn_fmed3f(c, -mx, mx);
  d = __builtin_amdgcn_fmed3f(d, -mx, mx);
  int r;
  if constexpr (FMT == TE_E4M3) {
    r = __builtin_amdgcn_cvt_pk_fp8_f32(a, b, 0, false);
    r = __builtin_amdgcn_cvt_pk_fp8_f32(c, d, r, true);
  } else {
    r = __builtin_amdgcn_cvt_pk_bf8_f32(a, b, 0, false);
    r = __builtin_amdgcn_cvt_pk_bf8_f32(c, d, r, true);
  }
  return (uint32_t)r;
}

// Current-scaling cast with the final reduction folded in: every workgroup
// reduces the partial maxima itself (a few KB from L2, issued after its own
// loads of x so the two overlap), derives the scale, and casts 4 chunks per
// thread; workgroup 0 writes amax, scale and scale_inv, and its thread 0 the
// n % 8 tail.  One launch fewer than final reduction + cast.
constexpr int kCastThreads = 256;
constexpr int kCastUnroll = 4;

template <int FMT>
__global__ __launch_bounds__(kCastThreads) void cast_current_kernel(const uint16_t* __restrict__ x, int64_t n,
                                                                   const uint32_t* __restrict__ partial, int nparts,
                                                                   uint8_t* __restrict__ q,
                                                                   float* __restrict__ amax_out,
                                                                   float* __restrict__ scale_out,
                                                                   float* __restrict__ scale_inv_out) {
  static_assert(kCastThreads == kAmaxThreads, "block_max reduces over kAmaxThreads lanes");
  const int64_t nchunks = n / 8;
  const int64_t base = (int64_t)blockIdx.x * (kCastThreads * kCastUnroll) + threadIdx.x;
  const uint4* xv = reinterpret_cast<const uint4*>(x);
  uint4 v[kCastUnroll];
#pragma unroll
  for (int u = 0; u < kCastUnroll; ++u) {
    const int64_t c = base + (int64_t)u * kCastThreads;
    v[u] = c < nchunks ? load_nt16(xv + c) : make_uint4(0, 0, 0, 0);
  }
  uint32_t m = 0;
  for (int i = threadIdx.x; i < nparts; i += kCastThreads) m = max(m, partial[i]);
  m = block_max(m);
  const float amax = bf16_bits_to_float(m);
  const float scale = current_scale<FMT>(amax);
  if (blockIdx.x == 0 && threadIdx.x == 0) {
    *amax_out = amax;
    *scale_out = scale;
    *scale_inv_out = (float)(1.0 / (double)scale);
  }
#pragma unroll
  for (int u = 0; u < kCastUnroll; ++u) {
    const int64_t c = base + (int64_t)u * kCastThreads;
    if (c < nchunks) {
      uint2 r;
      r.x = cast4<FMT>(v[u].x, v[u].y, scale);
      r.y = cast4<FMT>(v[u].z, v[u].w, scale);
      store_nt8(reinterpret_cast<uint2*>(q) + c, r);
    }
  }
  if (blockIdx.x == 0 && threadIdx.x == 0) {
    for (int64_t i = nchunks * 8; i < n; ++i) q[i] = (uint8_t)(cast4<FMT>(x[i], 0, scale) & 0xFFu);
  }
}

// Delayed scaling ("Getting Started" recipes: DelayedScaling with an amax
// history; "Workflow: ... Quickstart" Step 4).  One pass casts x with the
// scale the history has given so far and records per-workgroup maxima of
// |x| (x is read once); then one workgroup shifts the history (newest first),
// reduces it (max, or the most recent), and replaces the scale with
// fl32(fl32(fmt_max / r) / 2^margin) when r is positive and finite.
template <int FMT>
__global__ __launch_bounds__(kAmaxThreads) void cast_amax_kernel(const uint16_t* __restrict__ x, int64_t n,
                                                                 const float* __restrict__ scale_ptr,
                                                                 uint8_t* __restrict__ q,
                                                                 uint32_t* __restrict__ partial) {
  const float scale = *scale_ptr;
  const int64_t nchunks = n / 8;
  const uint4* xv = reinterpret_cast<const uint4*>(x);
  uint32_t m = 0;
  const int64_t stride = (int64_t)gridDim.x * kAmaxThreads * kAmaxUnroll;
  for (int64_t c0 = (int64_t)blockIdx.x * kAmaxThreads * kAmaxUnroll + threadIdx.x; c0 < nchunks; c0 += stride) {
    uint4 v[kAmaxUnroll];
#pragma unroll
    for (int u = 0; u < kAmaxUnroll; ++u) {
      const int64_t c = c0 + (int64_t)u * kAmaxThreads;
      v[u] = c < nchunks ? load_nt16(xv + c) : make_uint4(0, 0, 0, 0);
    }
#pragma unroll
    for (int u = 0; u < kAmaxUnroll; ++u) {
      const int64_t c = c0 + (int64_t)u * kAmaxThreads;
      if (c < nchunks) {
        m = max(m, absmax_bits8(v[u]));
        uint2 r;
        r.x = cast4<FMT>(v[u].x, v[u].y, scale);
        r.y = cast4<FMT>(v[u].z, v[u].w, scale);
        reinterpret_cast<uint2*>(q)[c] = r;
      }
    }
  }
  if (blockIdx.x == 0) {  // the n % 8 tail
    const int64_t i = nchunks * 8 + threadIdx.x;
    if (i < n) {
      const uint32_t h = x[i];
      m = max(m, h & 0x7FFFu);
      q[i] = (uint8_t)(cast4<FMT>(h, 0, scale) & 0xFFu);
    }
  }
  m = block_max(m);
  if (threadIdx.x == 0) partial[blockIdx.x] = m;
}

constexpr int kMaxHistory = 1024;

template <int FMT>
__global__ __launch_bounds__(kAmaxThreads) void delayed_update_kernel(const uint32_t* __restrict__ partial,
                                                                      int nparts, float* __restrict__ history,
                                                                      int len, int most_recent, int margin,
                                                                      float* __restrict__ scale,
                                                                      float* __restrict__ q_scale_inv) {
  // every global read first (history entries, the old scale, the partial maxima): one memory
  // round trip instead of three dependent ones
  float held[kMaxHistory / kAmaxThreads];
#pragma unroll
  for (int k = 0; k < kMaxHistory / kAmaxThreads; ++k) {
    const int i = threadIdx.x + k * kAmaxThreads;
    held[k] = i < len ? history[i] : 0.0f;
  }
  const float s_old = threadIdx.x == 0 ? *scale : 0.0f;
  uint32_t m = 0;
  for (int i = threadIdx.x; i < nparts; i += kAmaxThreads) m = max(m, partial[i]);
  m = block_max(m);
  const float amax = bf16_bits_to_float(m);
  // every wave has read block_max's result (its LDS is reused below) and every history entry
  // before any shifted write
  __syncthreads();
  uint32_t r = 0;  // max of the new history, over non-negative float bit patterns
#pragma unroll
  for (int k = 0; k < kMaxHistory / kAmaxThreads; ++k) {
    const int i = threadIdx.x + k * kAmaxThreads;
    if (i + 1 < len) {
      history[i + 1] = held[k];
      r = max(r, __float_as_uint(held[k]));
    }
  }
  r = block_max(r);
  if (threadIdx.x != 0) return;
  history[0] = amax;
  // over bit patterns (all entries are >= 0): a NaN sorts above inf and, like the
  // plain maximum, makes the result non-finite, so the scale is kept
  const float red = most_recent ? amax : __uint_as_float(max(__float_as_uint(amax), r));
  *q_scale_inv = (float)(1.0 / (double)s_old);  // the inverse of the scale the cast used
  if (red > 0.0f && red <= FLT_MAX) {
    // correctly rounded fp32 quotient (see current_scale), then an exact power-of-two division
    float s = (float)((double)FmtTraits<FMT>::max_value / (double)red);
    if (!(s <= FLT_MAX)) s = FLT_MAX;
    *scale = ldexpf(s, -margin);
  }
}

te_status launch_amax(const uint16_t* x, int64_t n, uint32_t* partial, int64_t blocks, bool nontemporal,
                      hipStream_t stream) {
  if (nontemporal)
    hipLaunchKernelGGL(amax_partial_kernel<true>, dim3((unsigned)blocks), dim3(kAmaxThreads), 0, stream, x, n,
                       partial);
  else
    hipLaunchKernelGGL(amax_partial_kernel<false>, dim3((unsigned)blocks), dim3(kAmaxThreads), 0, stream, x, n,
                       partial);
  return launch_status();
}

// The checks both current-scaling entry points share (everything but the
// partial-maxima buffer).
te_status check_cast_current(const uint16_t* x, int64_t n, te_dtype fmt, const uint8_t* q_out, const float* amax_out,
                             const float* scale_out, const float* scale_inv_out) {
  TE_REQUIRE(is_fp8(fmt), TE_ERR_DTYPE);
  TE_REQUIRE(n >= 0, TE_ERR_SHAPE);
  TE_REQUIRE(amax_out != nullptr && scale_out != nullptr && scale_inv_out != nullptr, TE_ERR_NULL);
  TE_REQUIRE(n == 0 || (x != nullptr && q_out != nullptr), TE_ERR_NULL);
  TE_REQUIRE(n == 0 || (aligned16(x) && aligned16(q_out)), TE_ERR_ALIGN);
  TE_REQUIRE(n / 8 / 256 < (int64_t)1 << 31, TE_ERR_SHAPE);
  return TE_OK;
}

// Stage one of the amax into `partial` (blocks entries), then the cast with
// the final reduction folded in.
te_status launch_cast_current(const uint16_t* x, int64_t n, te_dtype fmt, uint8_t* q_out, float* amax_out,
                              float* scale_out, float* scale_inv_out, uint32_t* partial, int64_t blocks,
                              hipStream_t stream) {
  if (launch_amax(x, n, partial, blocks, /*nontemporal=*/false, stream) != TE_OK) return TE_ERR_HIP;
  // at least one workgroup, which writes amax, scale and scale_inv (n = 0 included)
  int64_t grid = (n / 8 + kCastThreads * kCastUnroll - 1) / (kCastThreads * kCastUnroll);
  if (grid < 1) grid = 1;
  if (fmt == TE_E4M3)
    hipLaunchKernelGGL(cast_current_kernel<TE_E4M3>, dim3((unsigned)grid), dim3(kCastThreads), 0, stream, x, n,
                       partial, (int)blocks, q_out, amax_out, scale_out, scale_inv_out);
  else
    hipLaunchKernelGGL(cast_current_kernel<TE_E5M2>, dim3((unsigned)grid), dim3(kCastThreads), 0, stream, x, n,
                       partial, (int)blocks, q_out, amax_out, scale_out, scale_inv_out);
  return launch_status();
}

// Partial maxima of te_fp8_cast_current_scaling_noalloc, for callers that
// cannot allocate: one uint32 per amax workgroup of the cast, at most
// kCastAmaxBlocks (2 KB), in static device memory.  Every GPU the library
// runs on holds its own copy until the process ends; calls on one GPU share it
// (each call writes every entry it reads, so nothing needs clearing between
// calls).
constexpr int64_t kScratchPartials = kCastAmaxBlocks;
static __device__ __align__(256) uint32_t scratch[kScratchPartials];

// Device address of this GPU's copy of `scratch`, looked up once per device
// with that device current (in host code the array's name is only a
// host-side stand-in).  nullptr if the lookup fails.
uint32_t* scratch_partials() {
  static std::atomic<uint32_t*> cache[64];
  static std::mutex lookup;
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return nullptr;
  uint32_t* ptr = cache[dev].load(std::memory_order_acquire);
  if (ptr != nullptr) return ptr;
  std::lock_guard<std::mutex> guard(lookup);
  ptr = cache[dev].load(std::memory_order_acquire);
  if (ptr == nullptr) {
    void* addr = nullptr;
    if (hipGetSymbolAddress(&addr, HIP_SYMBOL(scratch)) != hipSuccess || addr == nullptr) return nullptr;
    ptr = static_cast<uint32_t*>(addr);
    cache[dev].store(ptr, std::memory_order_release);
  }
  return ptr;
}

}  // namespace
}  // namespace temx

using namespace temx;

extern "C" size_t te_amax_workspace_size(int64_t n) {
  if (n < 0) return 0;
  return (size_t)amax_blocks(n) * sizeof(uint32_t);
}

extern "C" te_status te_amax_reduce(const uint16_t* x, int64_t n, float* amax_out, void* workspace,
                                    size_t workspace_bytes, hipStream_t stream) {
  TE_REQUIRE(n >= 0, TE_ERR_SHAPE);
  TE_REQUIRE(amax_out != nullptr && workspace != nullptr, TE_ERR_NULL);
  TE_REQUIRE(n == 0 || x != nullptr, TE_ERR_NULL);
  TE_REQUIRE(n == 0 || aligned16(x), TE_ERR_ALIGN);
  TE_REQUIRE(((uintptr_t)workspace & 3u) == 0, TE_ERR_ALIGN);
  const int64_t blocks = amax_blocks(n);
  TE_REQUIRE(workspace_bytes >= (size_t)blocks * sizeof(uint32_t), TE_ERR_WORKSPACE);
  uint32_t* partial = static_cast<uint32_t*>(workspace);
  TE_REQUIRE(device_is_gfx950(), TE_ERR_ARCH);
  if (launch_amax(x, n, partial, blocks, /*nontemporal=*/true, stream) != TE_OK) return TE_ERR_HIP;
  hipLaunchKernelGGL(amax_final_kernel, dim3(1), dim3(kAmaxThreads), 0, stream, partial, (int)blocks, amax_out);
  return launch_status();
}

extern "C" te_status te_fp8_cast_current_scaling(const uint16_t* x, int64_t n, te_dtype fmt, uint8_t* q_out,
                                                 float* amax_out, float* scale_out, float* scale_inv_out,
                                                 void* workspace, size_t workspace_bytes, hipStream_t stream) {
  const te_status st = check_cast_current(x, n, fmt, q_out, amax_out, scale_out, scale_inv_out);
  if (st != TE_OK) return st;
  TE_REQUIRE(workspace != nullptr, TE_ERR_NULL);
  TE_REQUIRE(((uintptr_t)workspace & 3u) == 0, TE_ERR_ALIGN);
  const int64_t blocks = cast_amax_blocks(n);
  TE_REQUIRE(workspace_bytes >= (size_t)blocks * sizeof(uint32_t), TE_ERR_WORKSPACE);
  TE_REQUIRE(device_is_gfx950(), TE_ERR_ARCH);
  return launch_cast_current(x, n, fmt, q_out, amax_out, scale_out, scale_inv_out, static_cast<uint32_t*>(workspace),
                             blocks, stream);
}

extern "C" te_status te_fp8_cast_current_scaling_noalloc(const uint16_t* x, int64_t n, te_dtype fmt, uint8_t* q_out,
                                                         float* amax_out, float* scale_out, float* scale_inv_out,
                                                         hipStream_t stream) {
  const te_status st = check_cast_current(x, n, fmt, q_out, amax_out, scale_out, scale_inv_out);
  if (st != TE_OK) return st;
  const int64_t blocks = cast_amax_blocks(n);
  // the cast's amax grid is capped at kCastAmaxBlocks workgroups, so every n fits the scratch
  static_assert(kScratchPartials >= kCastAmaxBlocks, "one scratch entry per amax workgroup");
  TE_REQUIRE(blocks <= kScratchPartials, TE_ERR_WORKSPACE);
  TE_REQUIRE(device_is_gfx950(), TE_ERR_ARCH);
  uint32_t* partial = scratch_partials();
  TE_REQUIRE(partial != nullptr, TE_ERR_HIP);
  return launch_cast_current(x, n, fmt, q_out, amax_out, scale_out, scale_inv_out, partial, blocks, stream);
}

extern "C" te_status te_fp8_cast_delayed_scaling(const uint16_t* x, int64_t n, te_dtype fmt, uint8_t* q_out,
                                                 float* q_scale_inv_out, float* scale, float* amax_history,
                                                 int history_len, te_amax_algo algo, int margin, void* workspace,
                                                 size_t workspace_bytes, hipStream_t stream) {
  TE_REQUIRE(is_fp8(fmt), TE_ERR_DTYPE);
  TE_REQUIRE(algo == TE_AMAX_MAX || algo == TE_AMAX_MOST_RECENT, TE_ERR_VALUE);
  TE_REQUIRE(n >= 0 && history_len >= 1 && history_len <= kMaxHistory, TE_ERR_SHAPE);
  TE_REQUIRE(margin >= 0 && margin <= 64, TE_ERR_VALUE);
  TE_REQUIRE(q_scale_inv_out != nullptr && scale != nullptr && amax_history != nullptr && workspace != nullptr,
             TE_ERR_NULL);
  TE_REQUIRE(n == 0 || (x != nullptr && q_out != nullptr), TE_ERR_NULL);
  TE_REQUIRE(n == 0 || (aligned16(x) && aligned16(q_out)), TE_ERR_ALIGN);
  TE_REQUIRE(((uintptr_t)workspace & 3u) == 0, TE_ERR_ALIGN);
  TE_REQUIRE(((uintptr_t)scale & 3u) == 0 && ((uintptr_t)amax_history & 3u) == 0 &&
                 ((uintptr_t)q_scale_inv_out & 3u) == 0,
             TE_ERR_ALIGN);
  const int64_t blocks = amax_blocks(n);
  TE_REQUIRE(workspace_bytes >= (size_t)blocks * sizeof(uint32_t), TE_ERR_WORKSPACE);
  uint32_t* partial = static_cast<uint32_t*>(workspace);
  const int mr = algo == TE_AMAX_MOST_RECENT ? 1 : 0;
  TE_REQUIRE(device_is_gfx950(), TE_ERR_ARCH);
  if (fmt == TE_E4M3) {
    hipLaunchKernelGGL(cast_amax_kernel<TE_E4M3>, dim3((unsigned)blocks), dim3(kAmaxThreads), 0, stream, x, n, scale,
                       q_out, partial);
    if (launch_status() != TE_OK) return TE_ERR_HIP;
    hipLaunchKernelGGL(delayed_update_kernel<TE_E4M3>, dim3(1), dim3(kAmaxThreads), 0, stream, partial, (int)blocks,
                       amax_history, history_len, mr, margin, scale, q_scale_inv_out);
  } else {
    hipLaunchKernelGGL(cast_amax_kernel<TE_E5M2>, dim3((unsigned)blocks), dim3(kAmaxThreads), 0, stream, x, n, scale,
                       q_out, partial);
    if (launch_status() != TE_OK) return TE_ERR_HIP;
    hipLaunchKernelGGL(delayed_update_kernel<TE_E5M2>, dim3(1), dim3(kAmaxThreads), 0, stream, partial, (int)blocks,
                       amax_history, history_len, mr, margin, scale, q_scale_inv_out);
  }
  return launch_status();
}
