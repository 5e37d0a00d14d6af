// Issue-rate probe of the vector ALU on gfx950 (measurement only, not part of
// the scan library's ABI): how many float32 FMA lane-operations and how many
// v_exp_f32 lane-operations one MI355X completes per second, alone and mixed
// in the scan's ratio (one exp per four other operations). The scan's cost
// model in slots per element is built on these two rates.
//
// Every thread runs `iters` iterations of a fully unrolled body over 8
// independent dependency chains (enough to cover the VALU latency with 8 waves
// per SIMD), so the rate is issue-bound. The chains' results are written out
// so that nothing is removed by the compiler.
//
//   kind 0: 16 x 8 v_fma_f32 per iteration
//   kind 1: 16 x 8 v_exp_f32 per iteration (argument -|v|, so values stay finite)
//   kind 2: 16 x 8 (v_exp_f32 + 4 v_fma_f32) per iteration
//   kind 3: 16 x 8 v_fmac_f32 with a DPP quad-broadcast operand per iteration
//           (the form the scan's C contraction takes)
//
// Built into libssm_valu_probe.so; the benchmark's --micro mode times it.

#include <hip/hip_runtime.h>

#include <cstdint>

namespace {

constexpr int kUnroll = 16;
constexpr int kChains = 8;

template <int KIND>
__global__ __launch_bounds__(256) void valu_rate_kernel(float* out, int iters, float seed) {
  float v[kChains], w[kChains];
#pragma unroll
  for (int j = 0; j < kChains; ++j) {
    v[j] = seed + 1e-3f * static_cast<float>(threadIdx.x) + static_cast<float>(j);
    w[j] = 0.5f * v[j];
  }
  for (int i = 0; i < iters; ++i) {
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
#pragma unroll
      for (int j = 0; j < kChains; ++j) {
        if constexpr (KIND == 0) {
          v[j] = __builtin_fmaf(v[j], 0.9999f, 1e-4f);
        } else if constexpr (KIND == 1) {
          v[j] = __builtin_amdgcn_exp2f(-__builtin_fabsf(v[j]));
        } else if constexpr (KIND == 3) {
          // v += w[lane 0 of the quad] * w: the DPP operand is read, not written
          const float b = __builtin_bit_cast(
              float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, w[j]), 0, 0xf, 0xf, true));
          v[j] = __builtin_fmaf(b, 0.9999f, v[j]);
        } else {
          const float a = __builtin_amdgcn_exp2f(-__builtin_fabsf(v[j]));
          w[j] = __builtin_fmaf(w[j], 0.9999f, a);
          v[j] = __builtin_fmaf(a, w[j], 1e-4f);
          w[j] = __builtin_fmaf(w[j], v[j], -1e-4f);
          v[j] = __builtin_fmaf(v[j], 0.5f, w[j]);
        }
      }
    }
  }
  float s = 0.f;
#pragma unroll
  for (int j = 0; j < kChains; ++j) s += v[j] + w[j];
  out[static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x] = s;
}

}  // namespace

extern "C" {

// Operations of each kind per thread and iteration: FMA lane-ops, exp lane-ops.
int ssm_probe_valu_ops_per_iter(int kind, int* fma, int* exp) {
  if (!fma || !exp) return 1;
  switch (kind) {
    case 0: *fma = kUnroll * kChains; *exp = 0; return 0;
    case 1: *fma = 0; *exp = kUnroll * kChains; return 0;
    case 2: *fma = 4 * kUnroll * kChains; *exp = kUnroll * kChains; return 0;
    case 3: *fma = kUnroll * kChains; *exp = 0; return 0;
    default: return 1;
  }
}

// Enqueues one launch of `blocks` workgroups of 256 threads on `stream`;
// `out` is a device buffer of blocks * 256 floats. Returns 0 on success,
// 1 for bad arguments, 2 if the launch was rejected.
int ssm_probe_valu_launch(int kind, int blocks, int iters, float* out, void* stream) {
  if (!out || blocks <= 0 || iters <= 0 || kind < 0 || kind > 3) return 1;
  hipStream_t st = static_cast<hipStream_t>(stream);
  switch (kind) {
    case 0: hipLaunchKernelGGL(valu_rate_kernel<0>, dim3(blocks), dim3(256), 0, st, out, iters, 0.25f); break;
    case 1: hipLaunchKernelGGL(valu_rate_kernel<1>, dim3(blocks), dim3(256), 0, st, out, iters, 0.25f); break;
    case 2: hipLaunchKernelGGL(valu_rate_kernel<2>, dim3(blocks), dim3(256), 0, st, out, iters, 0.25f); break;
    default: hipLaunchKernelGGL(valu_rate_kernel<3>, dim3(blocks), dim3(256), 0, st, out, iters, 0.25f); break;
  }
  return hipGetLastError() == hipSuccess ? 0 : 2;
}

}  // extern "C"
