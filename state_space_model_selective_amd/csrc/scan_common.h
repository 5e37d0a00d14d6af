// Internal helpers shared by the forward and backward selective-scan
// kernels (not part of the public C ABI).
#ifndef SSM_SCAN_COMMON_H
#define SSM_SCAN_COMMON_H

#include <hip/hip_runtime.h>

#include <algorithm>
#include <cstdint>

// Internal linkage: each translation unit gets its own copy.
namespace {

constexpr float kLog2e = 1.4426950408889634f;

// ---------------------------------------------------------------------------
// element access: float32 or bfloat16 (uint16 bit pattern)
// ---------------------------------------------------------------------------
__device__ __forceinline__ float to_f32(float v) { return v; }
__device__ __forceinline__ float to_f32(uint16_t v) { return __uint_as_float(static_cast<uint32_t>(v) << 16); }

template <typename T>
__device__ __forceinline__ T from_f32(float v);
template <>
__device__ __forceinline__ float from_f32<float>(float v) { return v; }
template <>
__device__ __forceinline__ uint16_t from_f32<uint16_t>(float v) {
  // round to nearest even; NaN stays NaN
  uint32_t u = __float_as_uint(v);
  if ((u & 0x7fffffffu) > 0x7f800000u) return static_cast<uint16_t>((u >> 16) | 0x40u);
  u += 0x7fffu + ((u >> 16) & 1u);
  return static_cast<uint16_t>(u >> 16);
}

// ---------------------------------------------------------------------------
// 4-wide element access (16-byte float32 / 8-byte bfloat16 vectors).
// Prefetches keep the loaded bits (Raw) and widen them only when they are
// used: a conversion right after the load would make the wave wait for the
// load there, and the prefetch would no longer overlap the computation.
// ---------------------------------------------------------------------------
template <typename T>
struct Vec4;
template <>
struct Vec4<float> {
  using Raw = float4;
  static __device__ __forceinline__ Raw zero() { return make_float4(0.f, 0.f, 0.f, 0.f); }
  static __device__ __forceinline__ Raw load_raw(const float* p) { return *reinterpret_cast<const float4*>(p); }
  static __device__ __forceinline__ float4 widen(Raw r) { return r; }
  static __device__ __forceinline__ float4 load(const float* p) { return *reinterpret_cast<const float4*>(p); }
  static __device__ __forceinline__ void store(float* p, float4 v) { *reinterpret_cast<float4*>(p) = v; }
};
template <>
struct Vec4<uint16_t> {
  using Raw = uint2;
  static __device__ __forceinline__ Raw zero() { return make_uint2(0u, 0u); }
  static __device__ __forceinline__ Raw load_raw(const uint16_t* p) { return *reinterpret_cast<const uint2*>(p); }
  static __device__ __forceinline__ float4 widen(Raw u) {
    return make_float4(__uint_as_float(u.x << 16), __uint_as_float(u.x & 0xffff0000u),
                       __uint_as_float(u.y << 16), __uint_as_float(u.y & 0xffff0000u));
  }
  static __device__ __forceinline__ float4 load(const uint16_t* p) { return widen(load_raw(p)); }
  static __device__ __forceinline__ void store(uint16_t* p, float4 v) {
    uint2 u;
    u.x = static_cast<uint32_t>(from_f32<uint16_t>(v.x)) | (static_cast<uint32_t>(from_f32<uint16_t>(v.y)) << 16);
    u.y = static_cast<uint32_t>(from_f32<uint16_t>(v.z)) | (static_cast<uint32_t>(from_f32<uint16_t>(v.w)) << 16);
    *reinterpret_cast<uint2*>(p) = u;
  }
};

// ---------------------------------------------------------------------------
// Options of the Bi-Mamba2 forward ("Some questions of Bi-Mamba2 and Hydra",
// the MambaChunkScanCombinedFn.forward listing): the step size used is
// clamp(softplus?(d + bias), lo, hi), softplus(v) = v above 20, else
// log(1 + e^v) (as log1p(e^v) for accuracy at small e^v); the output gate is
// y z sigmoid(z). bias points at the channel's (or head's) bias, or is null.
// ---------------------------------------------------------------------------
// 1 / v from the hardware reciprocal (v_rcp_f32, within 1 ulp): an IEEE
// division costs about ten instructions more, on the staging threads'
// critical path.
__device__ __forceinline__ float rcp_fast(float v) { return __builtin_amdgcn_rcpf(v); }

// log(v) for a normal positive v: the hardware base-2 logarithm (v_log_f32)
// times ln 2, a few ulp. (The library logf adds a rescaling for denormal
// arguments and an extra-precise ln 2 product: a dozen more instructions,
// on the staging threads' critical path.)
__device__ __forceinline__ float log_fast(float v) { return __builtin_amdgcn_logf(v) * 0.6931471805599453f; }

// log(1 + u) for u >= 0 from the hardware logarithm, accurate to a few ulp:
// with w = 1 + u rounded, log(w) u / (w - 1) cancels the rounding of w
// (D. Goldberg, "What every computer scientist should know about
// floating-point arithmetic", 1991, section 4.1); u itself when w rounds to 1.
// (w >= 1 is never denormal.)
__device__ __forceinline__ float log1p_pos(float u) {
  const float w = 1.f + u;
  return w == 1.f ? u : log_fast(w) * (u * rcp_fast(w - 1.f));
}

// e^x - 1 from the hardware exponential and logarithm (W. Kahan's method:
// with v = e^x rounded, (v - 1) x / log(v) cancels the rounding of v); x
// itself when v rounds to 1, -1 when v rounds to 0. Used with x <= 0, where
// v in (0, 1]: v below the normal range makes (v - 1) round to -1 first.
__device__ __forceinline__ float expm1_fast(float x) {
  const float v = __expf(x);
  if (v == 1.f) return x;
  const float vm = v - 1.f;
  return vm == -1.f ? -1.f : vm * (x * rcp_fast(log_fast(v)));
}

__device__ __forceinline__ float map_step(float d, const float* bias, int softplus, float lo, float hi) {
  if (bias) d += *bias;
  if (softplus) d = d > 20.f ? d : log1p_pos(__expf(d));
  return fminf(fmaxf(d, lo), hi);
}

// z sigmoid(z) (where e^-z overflows, the reciprocal of the infinite
// denominator is 0 and so is the result, as with a division)
__device__ __forceinline__ float silu(float z) { return z * rcp_fast(1.f + __expf(-z)); }

// ---------------------------------------------------------------------------
// Cross-lane operands (DPP). Lane q of a 16-lane row holds B_t[q] (or
// C_t[q]); quad g of the row needs B_t[4g .. 4g+3]. quad_bcast<J> makes every
// lane of a quad read lane J of that quad. As a plain move the compiler folds
// it into the consuming multiply as a DPP source modifier (and inserts the
// wait states DPP needs). It does not fold it into v_fmac, so dot products
// with the quad's values issue v_fmac_f32_dpp themselves (dot_quad).
// ---------------------------------------------------------------------------
template <int J>
__device__ __forceinline__ float quad_bcast(float v) {
  return __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, v), J * 0x55, 0xf, 0xf, true));
}

// sum_j (lane j of this lane's quad's src) * h[j]: a dot product of the
// quad's 4 values of src (B_t or C_t of the lane's 4 states) with h, as one
// DPP multiply and three DPP fmacs behind a single s_nop 1 (a DPP read of a
// VGPR needs two wait states after a VALU write of it; src is not written
// inside the block, and the accumulator is not a DPP operand).
__device__ __forceinline__ float dot_quad(float src, const float (&h)[4]) {
  float s;
  asm("s_nop 1\n\t"
      "v_mul_f32_dpp %0, %1, %2 quad_perm:[0,0,0,0] row_mask:0xf bank_mask:0xf bound_ctrl:1\n\t"
      "v_fmac_f32_dpp %0, %1, %3 quad_perm:[1,1,1,1] row_mask:0xf bank_mask:0xf bound_ctrl:1\n\t"
      "v_fmac_f32_dpp %0, %1, %4 quad_perm:[2,2,2,2] row_mask:0xf bank_mask:0xf bound_ctrl:1\n\t"
      "v_fmac_f32_dpp %0, %1, %5 quad_perm:[3,3,3,3] row_mask:0xf bank_mask:0xf bound_ctrl:1"
      : "=&v"(s)
      : "v"(src), "v"(h[0]), "v"(h[1]), "v"(h[2]), "v"(h[3]));
  return s;
}

// Issue priority of this wave, rotating with the round. The workgroups that
// share a compute unit were dispatched in turns of one per CU, so workgroup
// blockIdx.x is in turn blockIdx.x / ncu; with priority (round + turn) mod 3
// the (up to) three workgroups of a CU take turns at the highest priority.
// Without it the oldest waves win every issue tie: the first workgroup on a
// CU finishes long before the third, which then runs alone at low occupancy
// (measured on the MI355X: 48, 57 and 69 us for the three workgroups of every
// CU at 8 x 1024 x 1536; 58-65 us with the rotation). Used only when every
// workgroup is resident at once (ncu > 0): when later workgroups wait for a
// slot, the staggered finish of oldest-first issue lets them start earlier.
__device__ __forceinline__ void rotate_priority(int64_t r, int ncu) {
  if (ncu <= 0) return;
  switch (static_cast<int>((r + blockIdx.x / ncu) % 3)) {
    case 0: __builtin_amdgcn_s_setprio(0); break;
    case 1: __builtin_amdgcn_s_setprio(1); break;
    default: __builtin_amdgcn_s_setprio(2); break;
  }
}

// ---------------------------------------------------------------------------
// host-side helpers
// ---------------------------------------------------------------------------
struct Range {
  uintptr_t lo, hi;  // [lo, hi)
};

bool overlap(Range a, Range b) { return a.lo < b.hi && b.lo < a.hi; }

bool mul_ok(int64_t a, int64_t b, int64_t* out) {
  if (a <= 0 || b <= 0) return false;
  if (a > INT64_MAX / b) return false;
  *out = a * b;
  return true;
}

// a * b for sizes that may be zero (empty tensors); false if either is
// negative or the product overflows
bool mul_nn(int64_t a, int64_t b, int64_t* out) {
  if (a < 0 || b < 0) return false;
  if (a > 0 && b > 0 && a > INT64_MAX / b) return false;
  *out = a * b;
  return true;
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

Range rng(const void* p, int64_t bytes) {
  uintptr_t lo = reinterpret_cast<uintptr_t>(p);
  return Range{lo, lo + static_cast<uintptr_t>(bytes)};
}

int device_cus() {
  int dev = 0, ncu = 0;
  if (hipGetDevice(&dev) != hipSuccess) return 0;
  if (hipDeviceGetAttribute(&ncu, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) return 0;
  return ncu;
}

// The compute-unit count for rotate_priority when a launch of nblk
// workgroups (at most three per CU) is resident at once, else 0.
int rotation_cus(int64_t nblk) {
  const int ncu = device_cus();
  return (ncu > 0 && nblk <= 3 * static_cast<int64_t>(ncu)) ? ncu : 0;
}

// Extra (dynamic) LDS per workgroup so that the workgroups spread evenly over
// the compute units. The dispatcher fills a CU up to its resource limit before
// using the next one, so 768 workgroups that fit 4 per CU would run on 192 of
// 256 CUs. Padding each workgroup's LDS lowers the per-CU limit to
// ceil(blocks / CUs) when that is below the natural limit.
size_t spread_lds(int64_t nblk, size_t lds_static, int max_per_cu) {
  int dev = 0, ncu = 0, lds_cu = 0;
  if (hipGetDevice(&dev) != hipSuccess) return 0;
  if (hipDeviceGetAttribute(&ncu, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || ncu <= 0) return 0;
  if (hipDeviceGetAttribute(&lds_cu, hipDeviceAttributeMaxSharedMemoryPerMultiprocessor, dev) != hipSuccess ||
      lds_cu <= 0)
    return 0;
  const int64_t natural = std::min<int64_t>(max_per_cu, lds_cu / static_cast<int64_t>(lds_static));
  const int64_t want = (nblk + ncu - 1) / ncu;
  if (want >= natural || want <= 0) return 0;
  // per-workgroup LDS in (lds_cu / (want + 1), lds_cu / want]
  size_t total = static_cast<size_t>(lds_cu / (want + 1)) + 1024;
  total = (total + 511) & ~static_cast<size_t>(511);
  if (total > static_cast<size_t>(lds_cu / want) || total <= lds_static) return 0;
  return total - lds_static;
}

// Clears the split-sequence workspace header and flags (a kernel rather than
// a memset, so the call stays safe to capture in a graph).
__global__ void zero_words_kernel(unsigned* p, int64_t n) {
  for (int64_t i = blockIdx.x * static_cast<int64_t>(blockDim.x) + threadIdx.x; i < n;
       i += static_cast<int64_t>(gridDim.x) * blockDim.x)
    p[i] = 0u;
}

// dst[i] = src ? src[i] : 0 for n 4-byte words (the outputs of an empty
// sequence: final states equal to the initial ones, zero gradients)
__global__ void fill_words_kernel(unsigned* dst, const unsigned* src, int64_t n) {
  for (int64_t i = blockIdx.x * static_cast<int64_t>(blockDim.x) + threadIdx.x; i < n;
       i += static_cast<int64_t>(gridDim.x) * blockDim.x)
    dst[i] = src ? src[i] : 0u;
}

// Enqueues fill_words_kernel over `bytes` bytes (a multiple of 4) when dst is
// set and bytes > 0; false if the launch failed.
bool fill_async(void* dst, const void* src, int64_t bytes, hipStream_t stream) {
  if (!dst || bytes <= 0) return true;
  const int64_t n = bytes / 4;
  const unsigned grid = static_cast<unsigned>(std::min<int64_t>((n + 255) / 256, 1024));
  hipLaunchKernelGGL(fill_words_kernel, dim3(grid), dim3(256), 0, stream, static_cast<unsigned*>(dst),
                     static_cast<const unsigned*>(src), n);
  return hipGetLastError() == hipSuccess;
}

}  // namespace

#endif  // SSM_SCAN_COMMON_H
