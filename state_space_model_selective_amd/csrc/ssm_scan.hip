// Selective scan for MI355X (gfx950): C-ABI entry points and HIP kernels.
//
// Operation (see include/ssm_scan.h for the full contract): for each batch
// row b, channel e and state n,
//   a_t = exp(delta_t A[e,n]),  h_t = a_t h_{t-1} + (delta_t x_t) B_t[n],
//   y_t = sum_n C_t[n] h_t[n] + D[e] x_t,
// the API of "scan output is different between sequential and parallel
// versions" (mamba.py issue 26, the test script's API comment), and the
// bidirectional sum of a forward and a reverse-time scan with shared weights
// plus D x ("Some questions of Bi-Mamba2 and Hydra", the author's first reply).

#include <hip/hip_runtime.h>

#include <cstdint>
#include <cstring>
#include <type_traits>

#include "ssm_scan.h"

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
// Sequential kernel: one lane per channel (b, e), all N states in registers,
// the whole sequence in time order. B_t and C_t are the same for every lane
// of a block (one block covers 64 channels of one batch row), so they are
// read with uniform (scalar) loads.
//
// mode 0: y = sum_n C h + D x                      (forward scan)
// mode 1: part = sum_n C g + D x, time reversed    (first half of bidir)
// mode 2: y = part + sum_n C h                     (second half of bidir)
// ---------------------------------------------------------------------------
template <typename T, int N>
__global__ __launch_bounds__(64) void scan_seq_kernel(const T* __restrict__ x, const T* __restrict__ dl,
                                                      const float* __restrict__ A, const T* __restrict__ Bm,
                                                      const T* __restrict__ Cm, const float* __restrict__ D,
                                                      T* y, float* part,
                                                      float* __restrict__ h_out, int64_t L, int64_t ED,
                                                      int64_t nblk_e, int mode) {
  const int64_t b = blockIdx.x / nblk_e;
  const int64_t e = (blockIdx.x % nblk_e) * 64 + threadIdx.x;
  const bool live = e < ED;
  const int64_t ec = live ? e : ED - 1;

  float A2[N], h[N];
#pragma unroll
  for (int n = 0; n < N; ++n) {
    A2[n] = A[ec * N + n] * kLog2e;
    h[n] = 0.0f;
  }
  const float Dv = D ? D[ec] : 0.0f;
  const bool rev = (mode == 1);

  for (int64_t s = 0; s < L; ++s) {
    const int64_t t = rev ? (L - 1 - s) : s;
    const int64_t ix = (b * L + t) * ED + ec;
    const int64_t ib = (b * L + t) * N;
    const float dt = to_f32(dl[ix]);
    const float xv = to_f32(x[ix]);
    const float dx = dt * xv;
    float acc = 0.0f;
#pragma unroll
    for (int n = 0; n < N; ++n) {
      const float a = __builtin_amdgcn_exp2f(dt * A2[n]);
      h[n] = __builtin_fmaf(a, h[n], dx * to_f32(Bm[ib + n]));
      acc = __builtin_fmaf(to_f32(Cm[ib + n]), h[n], acc);
    }
    if (live) {
      if (mode == 0) {
        y[ix] = from_f32<T>(acc + Dv * xv);
      } else if (mode == 1) {
        part[ix] = acc + Dv * xv;
      } else {
        y[ix] = from_f32<T>(part[ix] + acc);
      }
    }
  }
  if (h_out && live) {
#pragma unroll
    for (int n = 0; n < N; ++n) h_out[(b * ED + e) * N + n] = h[n];
  }
}

// ---------------------------------------------------------------------------
// host-side validation
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

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

struct Sizes {
  int64_t seq;     // Bs * L * ED
  int64_t bc;      // Bs * L * N
  int64_t state;   // Bs * ED * N
  int64_t elem;    // bytes per x/delta/B/C/y element
};

int check_sizes(int64_t Bs, int64_t L, int64_t ED, int64_t N, int dtype, Sizes* s) {
  if (Bs <= 0 || L <= 0 || ED <= 0 || N <= 0) return SSM_ERR_DIM;
  int64_t t;
  if (!mul_ok(Bs, L, &t) || !mul_ok(t, ED, &s->seq) || !mul_ok(t, N, &s->bc)) return SSM_ERR_DIM;
  if (!mul_ok(Bs, ED, &t) || !mul_ok(t, N, &s->state)) return SSM_ERR_DIM;
  if (s->seq > INT64_MAX / 8 || s->state > INT64_MAX / 8) return SSM_ERR_DIM;
  if (dtype != SSM_F32 && dtype != SSM_BF16) return SSM_ERR_UNSUPPORTED;
  if (N != 16) return SSM_ERR_UNSUPPORTED;
  s->elem = dtype == SSM_F32 ? 4 : 2;
  return SSM_OK;
}

size_t workspace_bytes(int64_t Bs, int64_t L, int64_t ED, int64_t N, int dtype, int bidir) {
  Sizes s;
  if (check_sizes(Bs, L, ED, N, dtype, &s) != SSM_OK) return 0;
  // the bidirectional bf16 scan keeps its reverse-time partial sums in float32
  if (bidir && dtype == SSM_BF16) return static_cast<size_t>(s.seq) * 4;
  return 0;
}

Range rng(const void* p, int64_t bytes) {
  uintptr_t lo = reinterpret_cast<uintptr_t>(p);
  return Range{lo, lo + static_cast<uintptr_t>(bytes)};
}

int validate(const void* x, const void* delta, const float* A, const void* B, const void* C, const float* D,
             const void* y, const float* h_last, const float* g_first, int64_t Bs, int64_t L, int64_t ED,
             int64_t N, int dtype, const void* ws, size_t ws_bytes, int bidir, Sizes* s) {
  if (!x || !delta || !A || !B || !C || !y) return SSM_ERR_NULL;
  int rc = check_sizes(Bs, L, ED, N, dtype, s);
  if (rc != SSM_OK) return rc;
  const void* ptrs[] = {x, delta, A, B, C, D, y, h_last, g_first, ws};
  for (const void* p : ptrs)
    if (p && !aligned16(p)) return SSM_ERR_UNSUPPORTED;
  size_t need = workspace_bytes(Bs, L, ED, N, dtype, bidir);
  if (need > 0 && (!ws || ws_bytes < need)) return SSM_ERR_WORKSPACE;

  Range in[] = {rng(x, s->seq * s->elem), rng(delta, s->seq * s->elem), rng(A, ED * N * 4),
                rng(B, s->bc * s->elem), rng(C, s->bc * s->elem), rng(D, D ? ED * 4 : 0)};
  Range out[4];
  int nout = 0;
  out[nout++] = rng(y, s->seq * s->elem);
  if (h_last) out[nout++] = rng(h_last, s->state * 4);
  if (g_first) out[nout++] = rng(g_first, s->state * 4);
  if (need > 0) out[nout++] = rng(ws, static_cast<int64_t>(need));
  for (int i = 0; i < nout; ++i) {
    for (const Range& r : in)
      if (r.hi > r.lo && overlap(out[i], r)) return SSM_ERR_ALIAS;
    for (int j = i + 1; j < nout; ++j)
      if (overlap(out[i], out[j])) return SSM_ERR_ALIAS;
  }
  return SSM_OK;
}

template <typename T>
int launch_scan(const void* x, const void* delta, const float* A, const void* B, const void* C, const float* D,
                void* y, float* h_last, float* g_first, int64_t Bs, int64_t L, int64_t ED, int bidir, void* ws,
                hipStream_t stream) {
  const int64_t nblk_e = (ED + 63) / 64;
  const int64_t nblk = Bs * nblk_e;
  if (nblk > INT32_MAX) return SSM_ERR_DIM;
  const T* xt = static_cast<const T*>(x);
  const T* dt = static_cast<const T*>(delta);
  const T* Bt = static_cast<const T*>(B);
  const T* Ct = static_cast<const T*>(C);
  T* yt = static_cast<T*>(y);
  if (!bidir) {
    hipLaunchKernelGGL((scan_seq_kernel<T, 16>), dim3(nblk), dim3(64), 0, stream, xt, dt, A, Bt, Ct, D, yt,
                       nullptr, h_last, L, ED, nblk_e, 0);
  } else {
    float* part = std::is_same<T, float>::value ? reinterpret_cast<float*>(y) : static_cast<float*>(ws);
    hipLaunchKernelGGL((scan_seq_kernel<T, 16>), dim3(nblk), dim3(64), 0, stream, xt, dt, A, Bt, Ct, D, yt,
                       part, g_first, L, ED, nblk_e, 1);
    hipLaunchKernelGGL((scan_seq_kernel<T, 16>), dim3(nblk), dim3(64), 0, stream, xt, dt, A, Bt, Ct, D, yt,
                       part, h_last, L, ED, nblk_e, 2);
  }
  return hipGetLastError() == hipSuccess ? SSM_OK : SSM_ERR_LAUNCH;
}

int run(const void* x, const void* delta, const float* A, const void* B, const void* C, const float* D, void* y,
        float* h_last, float* g_first, int64_t Bs, int64_t L, int64_t ED, int64_t N, int dtype, void* ws,
        size_t ws_bytes, void* stream, int bidir) {
  Sizes s;
  int rc = validate(x, delta, A, B, C, D, y, h_last, g_first, Bs, L, ED, N, dtype, ws, ws_bytes, bidir, &s);
  if (rc != SSM_OK) return rc;
  hipStream_t st = static_cast<hipStream_t>(stream);
  if (dtype == SSM_F32)
    return launch_scan<float>(x, delta, A, B, C, D, y, h_last, g_first, Bs, L, ED, bidir, ws, st);
  return launch_scan<uint16_t>(x, delta, A, B, C, D, y, h_last, g_first, Bs, L, ED, bidir, ws, st);
}

}  // namespace

extern "C" {

size_t ssm_scan_workspace_bytes(int64_t Bs, int64_t L, int64_t ED, int64_t N, int dtype, int bidir) {
  return workspace_bytes(Bs, L, ED, N, dtype, bidir);
}

int ssm_scan_fwd(const void* x, const void* delta, const float* A, const void* B, const void* C, const float* D,
                 void* y, float* h_last, int64_t Bs, int64_t L, int64_t ED, int64_t N, int dtype, void* workspace,
                 size_t workspace_bytes, void* stream) {
  return run(x, delta, A, B, C, D, y, h_last, nullptr, Bs, L, ED, N, dtype, workspace, workspace_bytes, stream, 0);
}

int ssm_scan_bidir_fwd(const void* x, const void* delta, const float* A, const void* B, const void* C,
                       const float* D, void* y, float* h_last, float* g_first, int64_t Bs, int64_t L, int64_t ED,
                       int64_t N, int dtype, void* workspace, size_t workspace_bytes, void* stream) {
  return run(x, delta, A, B, C, D, y, h_last, g_first, Bs, L, ED, N, dtype, workspace, workspace_bytes, stream, 1);
}

const char* ssm_status_str(int status) {
  switch (status) {
    case SSM_OK: return "ok";
    case SSM_ERR_NULL: return "a required pointer is NULL";
    case SSM_ERR_DIM: return "a dimension is not positive or the sizes overflow";
    case SSM_ERR_UNSUPPORTED: return "unsupported N or dtype, or a pointer not aligned to 16 bytes";
    case SSM_ERR_ALIAS: return "an output overlaps an input, another output or the workspace";
    case SSM_ERR_WORKSPACE: return "workspace missing or smaller than ssm_scan_workspace_bytes()";
    case SSM_ERR_LAUNCH: return "the HIP runtime rejected a kernel launch";
    default: return "unknown status";
  }
}

}  // extern "C"
