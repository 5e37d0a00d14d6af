// Multi-head (Mamba-2 / SSD) selective scan for MI355X (gfx950).
//
// For batch row b, head h (group g = h / (H / G)), head channel p and state n:
//   a_t = exp(dt[b,t,h] A[h])
//   S_t[p][n] = a_t S_{t-1}[p][n] + dt[b,t,h] x[b,t,h,p] B[b,t,g,n],   S_{-1} = h0 (or 0)
//   y[b,t,h,p] = sum_n C[b,t,g,n] S_t[p][n] + D[h] x[b,t,h,p]
// the layout of the chunked scan in "Some questions of Bi-Mamba2 and Hydra"
// (the MambaChunkScanCombinedFn listings: x (batch, seqlen, nheads, headdim),
// dt (batch, seqlen, nheads), one A per head, B and C per group).
//
// With one decay per head the scan over a chunk of Q steps is a few dense
// products (the chunked form of the scan): with cs_t = A sum_{r<=t} dt_r
// inside the chunk and S_in the state entering it,
//   Y   = M X + diag(e^{cs}) C S_in^T,     M[t][s] = (C_t . B_s) e^{cs_t - cs_s} dt_s  (s <= t)
//   S_out = e^{cs_end} S_in + sum_s X_s^T (e^{cs_end - cs_s} dt_s) B_s
// which the matrix cores compute. One workgroup owns one (batch row, head),
// keeps the head's 64 x N state in matrix-core accumulators for the whole
// sequence (the accumulators are also the operand of the output product)
// and walks the chunks in order; the next chunk's inputs are loaded into
// registers while the current one is computed (double-buffered LDS tiles).
//
// Two kernels: float32 inputs (ssd_fwd_kernel, below) on
// v_mfma_f32_16x16x4f32 with float32 operands and accumulation; bfloat16
// inputs (ssd_fwd_bf16_kernel, further down) on the bf16 matrix instruction
// with float32 accumulation and split operands.
//
// Matrix-core operand layout (16 x 16 x 4, one wave): lane l supplies
// A[l % 16][l / 16] and B[l / 16][l % 16]; result register r of lane l is
// D[4 (l / 16) + r][l % 16].
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <cstdint>
#include <type_traits>

#include "scan_common.h"
#include "ssm_scan.h"

namespace {

constexpr int kQ = 32;       // chunk length
constexpr int kP = 64;       // head channels (headdim)
constexpr int kWaves = 8;
// bf16 kernel: compute waves and staging waves
constexpr int kMainBf = 8;
constexpr int kStageBf = 4;
constexpr int kWavesBf = kMainBf + kStageBf;

template <typename T>
struct SsdArgs {
  const T* x;
  const T* dt;
  const float* A;
  const T* B;
  const T* C;
  const float* D;
  const float* h0;
  const float* g0;  // bidirectional: reverse state entering at t = L-1, or nullptr
  T* y;
  float* h_last;
  // bidirectional scan: float32 partial of the reverse direction, (Bs, L, H,
  // P) (may alias y for float32), and the reverse direction's final state
  float* part;
  float* g_first;
  // options: dt' = clamp(softplus?(dt + dt_bias[h]), dt_min, dt_max) when
  // dt_pre; the output (after D x and, bidirectional, both directions) times
  // z sigmoid(z) when z is set
  const float* dt_bias;
  int dt_softplus;
  int dt_pre;
  float dt_min, dt_max;
  const T* z;
  int64_t L, H, G;
  int nblocks;  // workgroups of the launch
  // split sequence: each (batch row, head) in nranges ranges of range_chunks
  // chunks; range j starts from the state folded in from ranges 0 .. j-1 of
  // its sweep (agg_S, agg_cs: per (range, batch row, head), a range's end
  // state from zero and A times its sum of step sizes)
  int nranges;
  int64_t range_chunks;
  int sweep_sel;   // -1: every sweep of the kernel; 0: the reverse sweep only; 1: the forward sweep only
  float* agg_S;    // [(j * Bs H + bh)][P][N] (the sweep's own array)
  double* agg_cs;  // [(j * Bs H + bh)]
};

// Workgroups are dealt to the 8 XCDs in turn (block i to XCD i mod 8). The
// (batch row, head) of block i is taken so that each XCD gets consecutive
// pairs, i.e. the heads of the same batch rows, which share B and C: those
// then come from the XCD's own L2 instead of every XCD fetching every row's.
// (Identity when the block count is not a multiple of 8.)
__device__ __forceinline__ int64_t xcd_local_block(int nblocks) {
  const int64_t blk = blockIdx.x;
  if (nblocks % 8 != 0) return blk;
  return (blk & 7) * (nblocks >> 3) + (blk >> 3);
}

// The (batch row, head) and, for a split sequence, the range of block i: in
// the order of xcd_local_block, range-major, so that the heads of a batch
// row's range (which share B and C) sit on one XCD.
struct SsdBlock {
  int bh, range, c0, c1;  // chunks [c0, c1) of the sweep (fewer than 2^31: L < 2^36)
};
template <typename T>
__device__ __forceinline__ SsdBlock ssd_block(const SsdArgs<T>& p) {
  SsdBlock r;
  const int blk = static_cast<int>(xcd_local_block(p.nblocks));
  const int nbh = p.nblocks / p.nranges;
  const int nchunks = static_cast<int>((p.L + 31) / 32);
  const int rc = static_cast<int>(p.range_chunks);
  r.range = __builtin_amdgcn_readfirstlane(blk / nbh);
  r.bh = __builtin_amdgcn_readfirstlane(blk % nbh);
  r.c0 = r.range * rc;
  r.c1 = r.c0 + rc < nchunks ? r.c0 + rc : nchunks;
  return r;
}

// Between the two passes of a split sequence: every range's end state from
// zero (agg_S) becomes, in place, the state entering that range: the sweep's
// initial state (init: (Bs, H, P, N), or zero) folded through the ranges
// before it, s = e^{cs_i} s + S_i, in range order. One thread per state
// element of a (batch row, head).
__global__ void ssd_join_kernel(float* agg_S, const double* agg_cs, const float* init, int64_t nbh, int64_t nranges,
                                int64_t PN) {
  const int64_t i = blockIdx.x * static_cast<int64_t>(blockDim.x) + threadIdx.x;
  if (i >= nbh * PN) return;
  const int64_t bh = i / PN, e = i % PN;
  float run = init ? init[i] : 0.f;
  for (int64_t j = 0; j < nranges; ++j) {
    const int64_t slot = j * nbh + bh;
    const float own = agg_S[slot * PN + e];
    agg_S[slot * PN + e] = run;
    run = __builtin_fmaf(__expf(static_cast<float>(agg_cs[slot])), run, own);
  }
}

// step size of the head whose bias (or null) is given, after the options
template <typename T>
__device__ __forceinline__ float ssd_step(const SsdArgs<T>& p, float d, const float* bias) {
  return p.dt_pre ? map_step(d, bias, p.dt_softplus, p.dt_min, p.dt_max) : d;
}
// the same with the head's bias held in a register (0 when there is none)
template <typename T>
__device__ __forceinline__ float ssd_step_v(const SsdArgs<T>& p, float d, float bias) {
  if (!p.dt_pre) return d;
  if (p.dt_bias) d += bias;
  return map_step(d, nullptr, p.dt_softplus, p.dt_min, p.dt_max);
}

// gate of 4 consecutive head channels of the row at time t (zero-filled bits
// past L are never used)
template <typename T>
__device__ __forceinline__ typename Vec4<T>::Raw load_gate(const SsdArgs<T>& p, int tid, int64_t b, int64_t h,
                                                           int64_t t) {
  if (t + (tid >> 4) >= p.L) return Vec4<T>::zero();
  return Vec4<T>::load_raw(p.z + ((b * p.L + t + (tid >> 4)) * p.H + h) * kP + (tid & 15) * 4);
}

__device__ __forceinline__ float4 gated(float4 v, float4 z) {
  return make_float4(v.x * silu(z.x), v.y * silu(z.y), v.z * silu(z.z), v.w * silu(z.w));
}

// Time of step tau of a sweep: the forward sweep runs t = tau, the reverse
// sweep of the bidirectional scan t = L - 1 - tau (inputs read in place).
__device__ __forceinline__ int64_t sweep_time(int64_t tau, int64_t L, bool rev) { return rev ? L - 1 - tau : tau; }

template <int N>
struct alignas(16) SsdSmem {
  float X[2][kQ][kP + 16];   // x chunk, row padded so that 4 consecutive rows hit different banks
  float Bm[2][kQ][N + 4];    // B chunk
  float Cm[2][kQ][N + 4];    // C chunk
  // the inter-chunk output block (t-block, p-block) over one half of the
  // states, [p][t] within the block, from the wave that does not own it
  float Yx[2][4][16][20];
  float M[2][kQ][kQ + 4];    // masked, decayed C B^T: two halves of the sum over n
  float Y[kQ][kP + 4];       // output of the chunk before D x
  float dt[2][kQ];
  float cs[kQ];              // A * inclusive cumulative dt within the chunk
  float ecs[kQ];             // e^{cs_t}
  float w[kQ];               // e^{cs_end - cs_s} dt_s
  float cs_end;
};

typedef float f4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ f4 mfma4(float a, float b, f4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
}

// Loads of one chunk into registers (4 elements per task, raw bits) and their
// commit to LDS (widened there). Rows at or past L are zero (dt = 0: a = 1 and
// no input); their loads read the last row instead (always in bounds, no
// branch around the load), and the commit drops them.
template <typename T, int N>
struct SsdStager {
  using V = Vec4<T>;
  static constexpr int kXT = kQ * kP / 4 / (64 * kWaves);  // x tasks per thread
  static constexpr int kBT = kQ * N / 4 / (64 * kWaves);   // B (and C) tasks per thread
  typename V::Raw rx[kXT], rb[kBT], rc[kBT];
  T rdt;
  bool vx[kXT], vb[kBT], vdt;

  // rows tau0 .. tau0 + kQ - 1 of the sweep (rev: time L - 1 - tau)
  __device__ __forceinline__ void load(const SsdArgs<T>& p, int tid, int64_t b, int64_t h, int64_t g, int64_t tau0,
                                       bool rev) {
#pragma unroll
    for (int k = 0; k < kXT; ++k) {
      const int u = tid + k * 64 * kWaves, row = u / (kP / 4), c4 = (u % (kP / 4)) * 4;
      const int64_t tau = tau0 + row;
      vx[k] = tau < p.L;
      const int64_t t = sweep_time(vx[k] ? tau : p.L - 1, p.L, rev);
      rx[k] = V::load_raw(p.x + ((b * p.L + t) * p.H + h) * kP + c4);
    }
#pragma unroll
    for (int k = 0; k < kBT; ++k) {
      const int u = tid + k * 64 * kWaves, row = u / (N / 4), c4 = (u % (N / 4)) * 4;
      const int64_t tau = tau0 + row;
      vb[k] = tau < p.L;
      const int64_t off = ((b * p.L + sweep_time(vb[k] ? tau : p.L - 1, p.L, rev)) * p.G + g) * N + c4;
      rb[k] = V::load_raw(p.B + off);
      rc[k] = V::load_raw(p.C + off);
    }
    const int64_t td = tau0 + (tid & (kQ - 1));
    vdt = tid < kQ && td < p.L;
    rdt = p.dt[(b * p.L + sweep_time(td < p.L ? td : p.L - 1, p.L, rev)) * p.H + h];
  }

  __device__ __forceinline__ void commit(SsdSmem<N>& sm, int buf, int tid) const {
    const float4 z = make_float4(0.f, 0.f, 0.f, 0.f);
#pragma unroll
    for (int k = 0; k < kXT; ++k) {
      const int u = tid + k * 64 * kWaves, row = u / (kP / 4), c4 = (u % (kP / 4)) * 4;
      *reinterpret_cast<float4*>(&sm.X[buf][row][c4]) = vx[k] ? V::widen(rx[k]) : z;
    }
#pragma unroll
    for (int k = 0; k < kBT; ++k) {
      const int u = tid + k * 64 * kWaves, row = u / (N / 4), c4 = (u % (N / 4)) * 4;
      *reinterpret_cast<float4*>(&sm.Bm[buf][row][c4]) = vb[k] ? V::widen(rb[k]) : z;
      *reinterpret_cast<float4*>(&sm.Cm[buf][row][c4]) = vb[k] ? V::widen(rc[k]) : z;
    }
    if (tid < kQ) sm.dt[buf][tid] = vdt ? to_f32(rdt) : 0.f;
  }
};

// AGG: the first pass of a split sequence (the ranges' end states from zero
// and their decays; no output).
template <typename T, int N, bool BIDIR, bool GATE, bool AGG = false>
__global__ __launch_bounds__(64 * kWaves) void ssd_fwd_kernel(const SsdArgs<T> p) {
  static_assert(kQ == 32 && kP == 64 && kWaves == 8, "work split below assumes these sizes");
  static_assert(N == 64 || N == 128, "state sizes");
  static_assert(!(AGG && (BIDIR || GATE)), "the aggregate pass runs one sweep, no gate");
  constexpr int NTL = N / 32;         // state tiles per wave (16 states each)

  __shared__ SsdSmem<N> sm;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int li = lane & 15, lk = lane >> 4;  // operand row / column and k index
  const SsdBlock blk = ssd_block(p);
  const int64_t bh = blk.bh;
  const int64_t b = bh / p.H, h = bh % p.H;
  const int64_t g = h / (p.H / p.G);
  const float Ah = p.A[h];
  const float Dh = p.D ? p.D[h] : 0.f;
  const float* const bias = p.dt_bias ? p.dt_bias + h : nullptr;

  // output block of this wave: t-block ytb (16 steps) x head-channel block
  // ypb. The wave's state: head channels p = 16 ypb .. 16 ypb + 15, states n
  // in half ytb of N, as NTL accumulator tiles S[n][p] (n the row): register
  // r of lane (li, lk) in tile k is n = N/2 ytb + 16 k + 4 lk + r, p = 16 ypb
  // + li. Register r of a tile is then, as it stands, the operand B (k = n,
  // column p) of one 16 x 16 x 4 product over n, so C S^T takes the state
  // from the accumulators and no copy of it goes through LDS.
  const int ytb = wave >> 2, ypb = wave & 3;
  const int pp = 16 * ypb + li;
  auto tile_n0 = [&](int k) { return (N / 2) * ytb + 16 * k + 4 * lk; };
  // C B^T task: causal block (0,0), (1,0) or (1,1), half of the sum over n
  const int mblk = wave >> 1, mhalf = wave & 1;
  const int mtb = mblk == 0 ? 0 : 1, msb = mblk == 2 ? 1 : 0;

  // BIDIR: a reverse sweep (zero initial state, no D x) storing a float32
  // partial, then the forward sweep adding it (a split sequence runs them in
  // separate launches: sweep_sel)
  for (int sweep = 0; sweep < (BIDIR ? 2 : 1); ++sweep) {
  if (BIDIR && p.sweep_sel >= 0 && sweep != p.sweep_sel) continue;  // (uniform)
  const bool rev = BIDIR ? sweep == 0 : p.sweep_sel == 0;
  const float* const init = rev ? p.g0 : p.h0;  // the sweep's entering state (null: zero)
  f4 st[NTL];
#pragma unroll
  for (int k = 0; k < NTL; ++k) {
    float4 v = make_float4(0.f, 0.f, 0.f, 0.f);
    if (!AGG) {
      // a range of a split sequence starts from its joined entering state
      if (p.nranges > 1)
        v = *reinterpret_cast<const float4*>(
            p.agg_S + ((blk.range * (p.nblocks / p.nranges) + bh) * kP + pp) * N + tile_n0(k));
      else if (init)
        v = *reinterpret_cast<const float4*>(init + ((b * p.H + h) * kP + pp) * N + tile_n0(k));
    }
    st[k][0] = v.x, st[k][1] = v.y, st[k][2] = v.z, st[k][3] = v.w;
  }
  double cs_sum = 0.0;  // AGG: A times the range's sum of step sizes (thread 0)

  SsdStager<T, N> stg;
  stg.load(p, tid, b, h, g, blk.c0 * kQ, rev);
  stg.commit(sm, 0, tid);
  __syncthreads();

  for (int64_t c = blk.c0; c < blk.c1; ++c) {
    const int cur = (c - blk.c0) & 1;
    const int64_t t0 = c * kQ;  // first step of the chunk in the sweep's order
    // decay of the chunk: cs_t, e^{cs_t}, the state-update weights (ahead of
    // the next chunk's loads, whose registers are live from there on)
    if (wave == 0 && lane < kQ) {
      // the step sizes after the options, in place (rows past L keep 0; the
      // wave's LDS accesses stay in order, so the reads below see them)
      if (p.dt_pre && t0 + lane < p.L) sm.dt[cur][lane] = ssd_step(p, sm.dt[cur][lane], bias);
      float s = 0.f, tot = 0.f;
#pragma unroll
      for (int r = 0; r < kQ; ++r) {
        const float v = sm.dt[cur][r];
        tot += v;
        s += r <= lane ? v : 0.f;
      }
      const float cst = Ah * s, cse = Ah * tot;
      sm.cs[lane] = cst;
      sm.ecs[lane] = __expf(cst);
      sm.w[lane] = __expf(cse - cst) * sm.dt[cur][lane];
      if (lane == 0) sm.cs_end = cse;
    }
    if (c + 1 < blk.c1) stg.load(p, tid, b, h, g, t0 + kQ, rev);
    // forward sweep of the bidirectional scan: the reverse partial of this
    // chunk's output rows, for the store at the chunk's end
    float4 pv = make_float4(0.f, 0.f, 0.f, 0.f);
    if (BIDIR && !rev && t0 + (tid >> 4) < p.L)
      pv = *reinterpret_cast<const float4*>(p.part + ((b * p.L + t0 + (tid >> 4)) * p.H + h) * kP + (tid & 15) * 4);
    // the gate of the same rows (forward sweep only: the partial is ungated)
    typename Vec4<T>::Raw zr = Vec4<T>::zero();
    if (GATE && !rev) zr = load_gate(p, tid, b, h, t0);

    __syncthreads();
    if (AGG && tid == 0) cs_sum += static_cast<double>(sm.cs_end);

    // C B^T on the causal blocks, each half of the sum over n by one wave,
    // masked and decayed into M[half]
    if (!AGG && wave < 6) {
      // operands first (all LDS reads in flight together), then the products
      constexpr int K = N / 8;
      float ca[K], cb[K];
      const int n1 = mhalf * (N / 2);
#pragma unroll
      for (int j = 0; j < K; ++j) {
        ca[j] = sm.Cm[cur][16 * mtb + li][n1 + 4 * j + lk];
        cb[j] = sm.Bm[cur][16 * msb + li][n1 + 4 * j + lk];
      }
      __builtin_amdgcn_sched_barrier(0);  // keep every read ahead of the products
      f4 a0 = {0.f, 0.f, 0.f, 0.f}, a1 = a0;
#pragma unroll
      for (int j = 0; j < K; j += 2) {
        a0 = mfma4(ca[j], cb[j], a0);
        a1 = mfma4(ca[j + 1], cb[j + 1], a1);
      }
      const int s = 16 * msb + li;
      const float css = sm.cs[s], dts = sm.dt[cur][s];
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int t = 16 * mtb + 4 * lk + r;
        sm.M[mhalf][t][s] = s <= t ? (a0[r] + a1[r]) * __expf(sm.cs[t] - css) * dts : 0.f;
      }
    }

    // inter-chunk output diag(e^{cs}) C S_in^T over the wave's half of the
    // states, for both t-blocks: the wave keeps its own block and hands the
    // other to its partner (same p-block, other half) through LDS
    f4 y = {0.f, 0.f, 0.f, 0.f};
    if (!AGG) {
#pragma unroll
      for (int tb = 0; tb < 2; ++tb) {
        float4 ca[NTL];
#pragma unroll
        for (int k = 0; k < NTL; ++k) ca[k] = *reinterpret_cast<const float4*>(&sm.Cm[cur][16 * tb + li][tile_n0(k)]);
        f4 a0 = {0.f, 0.f, 0.f, 0.f}, a1 = a0;
#pragma unroll
        for (int k = 0; k < NTL; ++k) {
          a0 = mfma4(ca[k].x, st[k][0], a0);
          a1 = mfma4(ca[k].y, st[k][1], a1);
          a0 = mfma4(ca[k].z, st[k][2], a0);
          a1 = mfma4(ca[k].w, st[k][3], a1);
        }
        const float4 e = *reinterpret_cast<const float4*>(&sm.ecs[16 * tb + 4 * lk]);
        const f4 v = {(a0[0] + a1[0]) * e.x, (a0[1] + a1[1]) * e.y, (a0[2] + a1[2]) * e.z, (a0[3] + a1[3]) * e.w};
        if (tb == ytb) y = v;
        else *reinterpret_cast<float4*>(&sm.Yx[tb][ypb][li][4 * lk]) = make_float4(v[0], v[1], v[2], v[3]);
      }
    }
    __syncthreads();  // M and the partner's block complete
    if (!AGG) {
      const float4 o = *reinterpret_cast<const float4*>(&sm.Yx[ytb][ypb][li][4 * lk]);
      y[0] += o.x, y[1] += o.y, y[2] += o.z, y[3] += o.w;
    }

    // intra-chunk output M X (causal: s-blocks up to the t-block); the
    // t-block 0 waves use the first half of the operands only
    if (!AGG) {
      float ma[8], xb[8];
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const int s0 = 4 * j;
        ma[j] = sm.M[0][16 * ytb + li][s0 + lk] + sm.M[1][16 * ytb + li][s0 + lk];
        xb[j] = sm.X[cur][s0 + lk][16 * ypb + li];
      }
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int j = 0; j < 4; ++j) y = mfma4(ma[j], xb[j], y);
      if (ytb == 1) {
#pragma unroll
        for (int j = 4; j < 8; ++j) y = mfma4(ma[j], xb[j], y);
      }
    }
    if (!AGG) {
#pragma unroll
      for (int r = 0; r < 4; ++r) sm.Y[16 * ytb + 4 * lk + r][16 * ypb + li] = y[r];
    }

    // state update S^T = e^{cs_end} S^T + B^T (w X) for the wave's tiles:
    // operand A B[s][n] (row n of the tile: 16 k + li of its half), operand
    // B w_s X[s][p]
    const float dec = __expf(sm.cs_end);
#pragma unroll
    for (int k = 0; k < NTL; ++k) st[k] *= dec;
    {
      float bo[kQ / 4][NTL], xa[kQ / 4];
#pragma unroll
      for (int j = 0; j < kQ / 4; ++j) {
        const int s0 = 4 * j;
        xa[j] = sm.X[cur][s0 + lk][pp] * sm.w[s0 + lk];
#pragma unroll
        for (int k = 0; k < NTL; ++k) bo[j][k] = sm.Bm[cur][s0 + lk][(N / 2) * ytb + 16 * k + li];
      }
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int j = 0; j < kQ / 4; ++j)
#pragma unroll
        for (int k = 0; k < NTL; ++k) st[k] = mfma4(bo[j][k], xa[j], st[k]);
    }
    __syncthreads();  // every read of this chunk's tiles and of the exchange is done; Y complete
    // the next chunk's tiles (waits for its loads), then this chunk's output:
    // the store is the last memory operation of the chunk, so no later wait
    // for the loads has to wait for it as well
    if (c + 1 < blk.c1) stg.commit(sm, cur ^ 1, tid);
    if (!AGG) {
      // 4 consecutive head channels per thread: y + D x (+ the reverse
      // partial) -> y, or the reverse sweep's partial -> part
      const int t = tid >> 4, c4 = (tid & 15) * 4;
      if (t0 + t < p.L) {
        const float4 yv = *reinterpret_cast<const float4*>(&sm.Y[t][c4]);
        const int64_t row = (b * p.L + sweep_time(t0 + t, p.L, rev)) * p.H + h;
        if (rev) {
          *reinterpret_cast<float4*>(p.part + row * kP + c4) = yv;
        } else {
          const float4 xv = *reinterpret_cast<const float4*>(&sm.X[cur][t][c4]);
          float4 o = make_float4(yv.x + Dh * xv.x + pv.x, yv.y + Dh * xv.y + pv.y, yv.z + Dh * xv.z + pv.z,
                                 yv.w + Dh * xv.w + pv.w);
          if (GATE) o = gated(o, Vec4<T>::widen(zr));
          Vec4<T>::store(p.y + row * kP + c4, o);
        }
      }
    }
    __syncthreads();
  }

  if (AGG) {
    // the range's end state from zero and its decay exponent
    const int64_t slot = blk.range * (p.nblocks / p.nranges) + bh;
#pragma unroll
    for (int k = 0; k < NTL; ++k)
      *reinterpret_cast<float4*>(p.agg_S + (slot * kP + pp) * N + tile_n0(k)) =
          make_float4(st[k][0], st[k][1], st[k][2], st[k][3]);
    if (tid == 0) p.agg_cs[slot] = cs_sum;
  } else {
    float* const fin = rev ? p.g_first : p.h_last;
    if (fin && blk.range == p.nranges - 1) {
#pragma unroll
      for (int k = 0; k < NTL; ++k)
        *reinterpret_cast<float4*>(fin + ((b * p.H + h) * kP + pp) * N + tile_n0(k)) =
            make_float4(st[k][0], st[k][1], st[k][2], st[k][3]);
    }
  }
  }  // sweep
}

// ---------------------------------------------------------------------------
// bfloat16 inputs. The products take bf16 operands on the bf16 matrix
// instruction, v_mfma_f32_16x16x32_bf16 (float32 accumulation; 16 times the
// float32 instruction's rate). C, B and x are bf16 already and enter exactly.
// The float32 operands -- the decayed, masked C B^T, the state (kept float32
// in the accumulators, which are also its operand) and the decay-weighted x
// of the state update -- are split into a high and a low bf16 part, v = hi +
// lo with hi = bf16(v) and lo = bf16(v - hi) (round to nearest even), and
// each product takes both parts: the operand error is then below 2^-17 |v|,
// so the state and the output keep float32-level accuracy.
//
// Operand layout (16 x 16 x 32, one wave): lane l supplies the 8 consecutive
// k = 8 (l / 16) .. 8 (l / 16) + 7 of row l % 16 of A and of column l % 16 of
// B, i.e. one 16-byte read of a k-contiguous LDS row; result register r of
// lane l is D[4 (l / 16) + r][l % 16]. Products over the state index n read
// n-contiguous tiles (C[t][n], B[s][n]); products over the chunk's steps
// read M[t][s] as it is and x[s][p], B[s][n] by transposing reads. Two result
// tiles whose registers hold the state's n = 32 g + 8 (l / 16) + 0..3 and
// + 4..7 are together the operand B of a product over n with C[t][32 g ..]
// read as usual, so the state never leaves the registers.
//
// Twelve waves: eight compute waves own the state and the output blocks,
// run the products and store the output; four staging waves move data and
// form each chunk's masked C B^T, so that this work overlaps the products
// instead of adding to them. Two of the staging waves load and commit tiles
// (16-byte global loads into registers in phase 1, committed in phase 2);
// they issue no stores, so their waits for loads never wait for stores
// (both count in the same counter). Per chunk, two barriers:
//   phase 1  compute waves: diag(e^{cs}) C S_in^T over the wave's half of
//            the states for both 16-step blocks (one goes to LDS for the
//            wave that owns it), and the update of the wave's state tiles,
//            S^T = e^{cs_end} S^T + B^T (w X) (so that a lane holds 4
//            consecutive n of one p); loads of what the output adds (the
//            reverse partial, the gate).
//            Staging waves: the chunk's three causal 16 x 16 blocks of C B^T
//            (computed as B C^T so that a lane holds 4 consecutive s of one
//            t) -> masked, decayed M (bf16 pair); issue the loads of the
//            next chunk
//   phase 2  compute waves: the other half's C S_in^T block, M X, + D x
//            -> y (or the reverse sweep's float32 partial), stored from the
//            registers. Loading waves: commit the next chunk's tiles and form
//            its decays (the last loading wave: a prefix sum over the lanes
//            (DPP) of the step sizes it loaded)
// ---------------------------------------------------------------------------
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

__device__ __forceinline__ f4 mfma_bf16(uint4 a, uint4 b, f4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a), __builtin_bit_cast(bf16x8, b), c, 0,
                                                 0, 0);
}
__device__ __forceinline__ uint32_t pack_bf16(float lo, float hi) {
  const bf16x2 v = {static_cast<__bf16>(lo), static_cast<__bf16>(hi)};
  return __builtin_bit_cast(uint32_t, v);
}
__device__ __forceinline__ uint16_t bf16_bits(float v) { return __builtin_bit_cast(uint16_t, static_cast<__bf16>(v)); }
// v = hi + lo, hi = bf16(v), lo = bf16(v - hi)
__device__ __forceinline__ void split_bf16(float v, uint16_t& hi, uint16_t& lo) {
  const __bf16 h = static_cast<__bf16>(v);
  hi = __builtin_bit_cast(uint16_t, h);
  lo = bf16_bits(v - static_cast<float>(h));
}
__device__ __forceinline__ void split_pack_bf16(float a, float b, uint32_t& hi, uint32_t& lo) {
  hi = pack_bf16(a, b);
  // the high parts back as float32 from the packed pair (a shift and a mask)
  lo = pack_bf16(a - __uint_as_float(hi << 16), b - __uint_as_float(hi & 0xffff0000u));
}
__device__ __forceinline__ float bf_lo(uint32_t u) { return __uint_as_float(u << 16); }
// Transposing LDS read of 16-bit elements (gfx950): within each group of 16
// lanes, lane i receives as element j the element i % 4 of the 8 bytes that
// lane 4 j + i / 4 of its group addresses (checked on the GPU with a probe).
// So if lane 4 j + q addresses 4 consecutive columns 4 q .. 4 q + 3 of row
// r0 + j of a row-major tile, lane i receives column i of rows r0 .. r0 + 3:
// a k-contiguous operand read from a tile stored the other way round.
typedef short v4i16 __attribute__((ext_vector_type(4)));
__device__ __forceinline__ uint2 read_tr16(const uint16_t* p) {
  const v4i16 v = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
      (__attribute__((address_space(3))) v4i16*)(const_cast<uint16_t*>(p)));
  return __builtin_bit_cast(uint2, v);
}
__device__ __forceinline__ float bf_hi(uint32_t u) { return __uint_as_float(u & 0xffff0000u); }

template <int N>
struct alignas(16) SsdSmemBf {
  // Row pitches (elements). With lanes on rows and 16-byte column blocks, a
  // 16-byte read is free of bank conflicts when the pitch in bytes is 32 mod
  // 64, an 8-byte access when it is 16 mod 64 (measured on gfx950): C is
  // only read and written 16 bytes at a time; B and x also take 8-byte
  // transposing reads.
  static constexpr int NPC = N + 16;  // C
  static constexpr int NP = N + 8;    // B
  static constexpr int TP = kQ + 8;   // the s-contiguous tiles
  static constexpr int XP = kP + 8;   // x
  uint16_t C[2][kQ][NPC];  // C chunk [t][n]
  uint16_t B[2][kQ][NP];   // B chunk [s][n]
  uint16_t X[2][kQ][XP];   // x chunk [s][p]
  uint16_t M[2][2][kQ][TP];  // masked, decayed C B^T [t][s] by chunk parity: high, low part
  // the inter-chunk output block (t-block, p-block) over one half of the
  // states, [p][t] within the block, from the wave that does not own it
  float Yx[2][4][16][24];
  float dt[2][kQ];
  float cs[2][kQ];         // A * inclusive cumulative dt within the chunk
  float ecs[2][kQ];        // e^{cs_t}
  float w[2][kQ];          // e^{cs_end - cs_s} dt_s
  float cs_end[2];
};

template <int N, int NT>
struct SsdStagerBf {
  static constexpr int kXT = kQ * kP / 8 / NT;  // x tasks (8 head channels of a row) per loading thread
  static constexpr int kBT = kQ * N / 8 / NT;   // B (and C) tasks (8 states of a row) per loading thread
  static constexpr int kDtWave = NT / 64 - 1;   // the loading wave whose lanes 0 .. kQ-1 load the step sizes
  static constexpr int kBRows = NT / (N / 8);   // rows between a thread's B tasks
  static_assert(NT % kQ == 0 && NT % (N / 8) == 0 && kXT >= 1 && kBT >= 1, "task split");
  uint4 rx[kXT], rb[kBT], rc[kBT];
  uint16_t rdt;
  bool vx, vb[kBT], vdt;
  // element offsets of the thread's first task rows in the next chunk to
  // load; sbr: from one B row to the next in the sweep's order (negative in
  // a reverse sweep); sx, sb, sd: from one chunk to the next
  int64_t ox, ob, od;
  int64_t sbr, sx, sb, sd;

  // the first chunk to load starts at sweep row tau0 (st: the loading
  // thread's index, 0 .. NT-1). Task k of x is row st % kQ, head channels
  // 8 (st / kQ + k NT / kQ) ..; task k of B and C is row st / (N / 8) +
  // k kBRows, states 8 (st % (N / 8)) ..
  __device__ __forceinline__ void init(const SsdArgs<uint16_t>& p, int st, int64_t b, int64_t h, int64_t g,
                                       int64_t tau0, bool rev) {
    const int64_t dir = rev ? -1 : 1;
    ox = ((b * p.L + sweep_time(tau0 + st % kQ, p.L, rev)) * p.H + h) * kP + (st / kQ) * 8;
    ob = ((b * p.L + sweep_time(tau0 + st / (N / 8), p.L, rev)) * p.G + g) * N + (st % (N / 8)) * 8;
    od = (b * p.L + sweep_time(tau0 + (st & (kQ - 1)), p.L, rev)) * p.H + h;
    sbr = dir * p.G * N;
    sx = dir * kQ * p.H * kP;
    sb = kQ * sbr;
    sd = dir * kQ * p.H;
  }

  // the chunk of sweep rows tau0 .. tau0 + kQ - 1 (the next one after the
  // previous load); rows at or past L are not read
  __device__ __forceinline__ void load(const SsdArgs<uint16_t>& p, int st, int64_t tau0) {
    vx = tau0 + st % kQ < p.L;
#pragma unroll
    for (int k = 0; k < kXT; ++k)
      rx[k] = vx ? *reinterpret_cast<const uint4*>(p.x + ox + k * (NT / kQ) * 8) : make_uint4(0u, 0u, 0u, 0u);
    ox += sx;
#pragma unroll
    for (int k = 0; k < kBT; ++k) {
      vb[k] = tau0 + st / (N / 8) + k * kBRows < p.L;
      const int64_t off = ob + k * kBRows * sbr;
      rb[k] = vb[k] ? *reinterpret_cast<const uint4*>(p.B + off) : make_uint4(0u, 0u, 0u, 0u);
      rc[k] = vb[k] ? *reinterpret_cast<const uint4*>(p.C + off) : make_uint4(0u, 0u, 0u, 0u);
    }
    ob += sb;
    vdt = (st >> 6) == kDtWave && (st & 63) < kQ && tau0 + (st & (kQ - 1)) < p.L;
    rdt = vdt ? p.dt[od] : uint16_t{0};
    od += sd;
  }

  // step size of this lane's row (zero past L or outside the dt task)
  // (rows past L keep dt = 0 whatever the options would make of it)
  __device__ __forceinline__ float dt_value(const SsdArgs<uint16_t>& p, float bias) const {
    return vdt ? ssd_step_v(p, to_f32(rdt), bias) : 0.f;
  }

  // rows at or past L are zero (dt = 0: a = 1 and no input)
  __device__ __forceinline__ void commit(const SsdArgs<uint16_t>& p, float bias, SsdSmemBf<N>& sm, int buf,
                                         int st) const {
#pragma unroll
    for (int k = 0; k < kXT; ++k) {
      const int row = st % kQ, c8 = (st / kQ + k * (NT / kQ)) * 8;
      *reinterpret_cast<uint4*>(&sm.X[buf][row][c8]) = rx[k];
    }
#pragma unroll
    for (int k = 0; k < kBT; ++k) {
      const int row = st / (N / 8) + k * kBRows, c8 = (st % (N / 8)) * 8;
      *reinterpret_cast<uint4*>(&sm.B[buf][row][c8]) = rb[k];
      *reinterpret_cast<uint4*>(&sm.C[buf][row][c8]) = rc[k];
    }
    if ((st >> 6) == kDtWave && (st & 63) < kQ) sm.dt[buf][st & 63] = dt_value(p, bias);
  }
};

// v summed over lanes 0 .. lane of each half wave (lanes 0..31 and 32..63):
// row shifts within the 16-lane rows, then row 1 (3) adds lane 15 (47)
template <int CTRL, int ROWS>
__device__ __forceinline__ float dpp_shifted(float x) {
  return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), CTRL, ROWS, 0xf, true));
}
__device__ __forceinline__ float lane_prefix_sum32(float v) {
  v += dpp_shifted<0x111, 0xf>(v);  // row_shr:1
  v += dpp_shifted<0x112, 0xf>(v);  // row_shr:2
  v += dpp_shifted<0x114, 0xf>(v);  // row_shr:4
  v += dpp_shifted<0x118, 0xf>(v);  // row_shr:8
  v += dpp_shifted<0x142, 0xa>(v);  // row_bcast:15 into rows 1 and 3
  return v;
}

// cs, e^{cs}, w and cs_end of the chunk in buffer buf, by the wave whose lanes
// 0 .. kQ-1 hold the chunk's step sizes (zero past L)
template <int N>
__device__ __forceinline__ void chunk_decay(SsdSmemBf<N>& sm, int buf, float Ah, int lane, float dtv) {
  const float incl = lane_prefix_sum32(dtv);
  const float tot = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, incl), kQ - 1));
  if (lane < kQ) {
    const float cst = Ah * incl, cse = Ah * tot;
    sm.cs[buf][lane] = cst;
    sm.ecs[buf][lane] = __expf(cst);
    sm.w[buf][lane] = __expf(cse - cst) * dtv;
    if (lane == 0) sm.cs_end[buf] = cse;
  }
}

// One sweep of the bf16 kernel over the chunks [blk.c0, blk.c1) of a
// (batch row, head): REV runs in decreasing time (chunk k of the sweep holds
// times L-1-32k .. L-32-32k) from g0, else in increasing time from h0.
template <int N, bool BIDIR, bool GATE, bool AGG, bool REV>
__device__ __forceinline__ void ssd_bf16_sweep(const SsdArgs<uint16_t>& p, SsdSmemBf<N>& sm, const SsdBlock& blk,
                                               float Dfwd, float bias) {
  constexpr int KN = N / 32;  // products over n: instructions per 16 x 16 block
  constexpr bool rev = REV;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int li = lane & 15, lk = lane >> 4;
  const int64_t bh = blk.bh;
  const int64_t b = bh / p.H, h = bh % p.H;
  const int64_t g = h / (p.H / p.G);
  const float Ah = p.A[h];
  const int64_t c0 = blk.c0, c1 = blk.c1;
  const float* const init = rev ? p.g0 : p.h0;  // the sweep's entering state (null: zero)
  const float Dh = rev ? 0.f : Dfwd;

  // Both roles run the same chunk loop with the same two barriers per chunk.
  if (wave < kMainBf) {
    // ================= compute waves =================
    // Wave (pb, nh) owns the state columns p = 16 pb .. 16 pb + 15 for half nh
    // of the states n, in accumulators, and the output block (t-block nh,
    // p-block pb). State tile k = 2 kg + ab: register r of lane (li, lk) is
    // S[n][p], p = 16 pb + li, n = N/2 nh + 32 kg + 8 lk + 4 ab + r. Its two
    // tiles of group kg, read as one register row, are then the operand B
    // (k = n, column p) of a product over n: lane (li, lk) holds n = 32 kg' +
    // 8 lk .. 8 lk + 7, the same k order as a 16-byte read of C[t][n]. The
    // state is its own operand: no copy of it goes through LDS.
    constexpr int KG = N / 64;    // 32-state groups per half
    constexpr int NTL = 2 * KG;   // state tiles per wave
    const int pb = wave & 3, nh = wave >> 2;
    const int pp = 16 * pb + li;
    auto tile_n0 = [&](int k) { return (N / 2) * nh + 32 * (k >> 1) + 8 * lk + 4 * (k & 1); };

    f4 st[NTL];
#pragma unroll
    for (int k = 0; k < NTL; ++k) {
      const int n0 = tile_n0(k);
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        float v = 0.f;
        if (!AGG) {
          // a range of a split sequence starts from its joined entering state
          if (p.nranges > 1) v = p.agg_S[((blk.range * (p.nblocks / p.nranges) + bh) * kP + pp) * N + n0 + r];
          else if (init) v = init[((b * p.H + h) * kP + pp) * N + n0 + r];
        }
        st[k][r] = v;
      }
    }
    double cs_sum = 0.0;  // AGG: A times the range's sum of step sizes (thread 0)
    // what the output of chunk cc adds (the reverse partial, the gate of the
    // lane's rows), into pvn / zn
    float pvn[4] = {0.f, 0.f, 0.f, 0.f}, zn[4] = {0.f, 0.f, 0.f, 0.f};
    auto load_adds = [&](int64_t cc) {
      if constexpr (!AGG && !REV && (BIDIR || GATE)) {
        const int64_t t = cc * kQ + 16 * nh + 4 * lk;
#pragma unroll
        for (int r = 0; r < 4; ++r)
          if (t + r < p.L) {
            const int64_t o = ((b * p.L + t + r) * p.H + h) * kP + pp;
            if (BIDIR) pvn[r] = p.part[o];
            if (GATE) zn[r] = to_f32(p.z[o]);
          }
      }
    };
    load_adds(c0);
    __syncthreads();

    for (int64_t c = c0; c < c1; ++c) {
      const int cur = (c - c0) & 1;
      // ---- phase 1 ----
      if (AGG && tid == 0) cs_sum += static_cast<double>(sm.cs_end[cur]);

      // the lane's 4 output rows: sweep rows tau0 .. tau0 + 3 (those before L),
      // head channel pp. The forward sweep of the bidirectional scan adds the
      // reverse sweep's partial of those rows and the gated form multiplies
      // by silu(z): both are loaded a chunk ahead of their use
      const int64_t tau0 = c * kQ + 16 * nh + 4 * lk;
      float pvv[4], zv[4];
#pragma unroll
      for (int r = 0; r < 4; ++r) pvv[r] = pvn[r], zv[r] = zn[r];
      if (c + 1 < c1) load_adds(c + 1);

      // inter-chunk output over this half of the states, both t-blocks:
      // diag(e^{cs}) C S_in^T; the partner wave (pb, 1 - nh) gets the block
      // it owns, this wave keeps its own
      f4 y = {0.f, 0.f, 0.f, 0.f};
      if (!AGG) {
        uint4 sh[KG], sl[KG];
#pragma unroll
        for (int kg = 0; kg < KG; ++kg) {
          uint32_t h0a, l0a, h1a, l1a, h0b, l0b, h1b, l1b;
          split_pack_bf16(st[2 * kg][0], st[2 * kg][1], h0a, l0a);
          split_pack_bf16(st[2 * kg][2], st[2 * kg][3], h1a, l1a);
          split_pack_bf16(st[2 * kg + 1][0], st[2 * kg + 1][1], h0b, l0b);
          split_pack_bf16(st[2 * kg + 1][2], st[2 * kg + 1][3], h1b, l1b);
          sh[kg] = make_uint4(h0a, h1a, h0b, h1b);
          sl[kg] = make_uint4(l0a, l1a, l0b, l1b);
        }
#pragma unroll
        for (int tb = 0; tb < 2; ++tb) {
          f4 a = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
          for (int kg = 0; kg < KG; ++kg) {
            const uint4 ca =
                *reinterpret_cast<const uint4*>(&sm.C[cur][16 * tb + li][(N / 2) * nh + 32 * kg + 8 * lk]);
            a = mfma_bf16(ca, sh[kg], a);
            a = mfma_bf16(ca, sl[kg], a);
          }
          const float4 e = *reinterpret_cast<const float4*>(&sm.ecs[cur][16 * tb + 4 * lk]);
          const f4 v = {a[0] * e.x, a[1] * e.y, a[2] * e.z, a[3] * e.w};
          if (tb == nh) y = v;
          else *reinterpret_cast<float4*>(&sm.Yx[tb][pb][li][4 * lk]) = make_float4(v[0], v[1], v[2], v[3]);
        }
      }

      // state update: S^T = e^{cs_end} S^T + B^T (w X), the weights on x
      uint2 xs0, xs1;  // x[8 lk .. 8 lk + 7][pp], the k slots of the products over s
      {
        const float dec = __expf(sm.cs_end[cur]);
#pragma unroll
        for (int k = 0; k < NTL; ++k) st[k] *= dec;
        // operand B: w_s X[s][p] for p = pp, s = 8 lk .. 8 lk + 7 (the k slots
        // of the lane), by two transposing reads of x (kept for M X below)
        xs0 = read_tr16(&sm.X[cur][8 * lk + (li >> 2)][16 * pb + 4 * (li & 3)]);
        xs1 = read_tr16(&sm.X[cur][8 * lk + 4 + (li >> 2)][16 * pb + 4 * (li & 3)]);
        const float4 w0 = *reinterpret_cast<const float4*>(&sm.w[cur][8 * lk]);
        const float4 w1 = *reinterpret_cast<const float4*>(&sm.w[cur][8 * lk + 4]);
        uint32_t xh[4], xl[4];
        split_pack_bf16(bf_lo(xs0.x) * w0.x, bf_hi(xs0.x) * w0.y, xh[0], xl[0]);
        split_pack_bf16(bf_lo(xs0.y) * w0.z, bf_hi(xs0.y) * w0.w, xh[1], xl[1]);
        split_pack_bf16(bf_lo(xs1.x) * w1.x, bf_hi(xs1.x) * w1.y, xh[2], xl[2]);
        split_pack_bf16(bf_lo(xs1.y) * w1.z, bf_hi(xs1.y) * w1.w, xh[3], xl[3]);
        const uint4 xoh = make_uint4(xh[0], xh[1], xh[2], xh[3]), xol = make_uint4(xl[0], xl[1], xl[2], xl[3]);
#pragma unroll
        for (int k = 0; k < NTL; ++k) {
          // operand A: B^T[n][s] = B[s][n] for the tile's rows, n = N/2 nh +
          // 32 kg + 8 (li / 4) + 4 ab + li % 4 for lane row li, by two
          // transposing reads (lane li's address: row 8 lk + li / 4 (+ 4),
          // columns from the tile row order's 4-column group li % 4)
          const int nc = (N / 2) * nh + 32 * (k >> 1) + 8 * (li & 3) + 4 * (k & 1);
          const uint2 b0 = read_tr16(&sm.B[cur][8 * lk + (li >> 2)][nc]);
          const uint2 b1 = read_tr16(&sm.B[cur][8 * lk + 4 + (li >> 2)][nc]);
          const uint4 ba = make_uint4(b0.x, b0.y, b1.x, b1.y);
          st[k] = mfma_bf16(ba, xoh, st[k]);
          st[k] = mfma_bf16(ba, xol, st[k]);
        }
      }
      __syncthreads();  // the next chunk's tiles committed; the partner's block written

      // ---- phase 2 ----
      if (!AGG) {
        // the partner's half of the inter-chunk block, then M X (M is zero
        // above the diagonal) and D x
        const float4 o = *reinterpret_cast<const float4*>(&sm.Yx[nh][pb][li][4 * lk]);
        y[0] += o.x, y[1] += o.y, y[2] += o.z, y[3] += o.w;
        const uint4 mh = *reinterpret_cast<const uint4*>(&sm.M[cur][0][16 * nh + li][8 * lk]);
        const uint4 ml = *reinterpret_cast<const uint4*>(&sm.M[cur][1][16 * nh + li][8 * lk]);
        const uint4 xb = make_uint4(xs0.x, xs0.y, xs1.x, xs1.y);
        y = mfma_bf16(mh, xb, y);
        y = mfma_bf16(ml, xb, y);
        // x[16 nh + 4 lk + r][pp] for the lane's output rows r
        const uint2 xv = read_tr16(&sm.X[cur][16 * nh + 4 * lk + (li >> 2)][16 * pb + 4 * (li & 3)]);
        y[0] += Dh * bf_lo(xv.x);
        y[1] += Dh * bf_hi(xv.x);
        y[2] += Dh * bf_lo(xv.y);
        y[3] += Dh * bf_hi(xv.y);
        // the wave stores its block itself: the reverse sweep its float32
        // partial, the forward sweep y (+ the partial, times the gate) rounded
        // once to bf16
#pragma unroll
        for (int r = 0; r < 4; ++r)
          if (tau0 + r < p.L) {
            const int64_t o = ((b * p.L + sweep_time(tau0 + r, p.L, rev)) * p.H + h) * kP + pp;
            if (rev) {
              p.part[o] = y[r];
            } else {
              float v = y[r] + pvv[r];
              if (GATE) v *= silu(zv[r]);
              p.y[o] = bf16_bits(v);
            }
          }
      }
      __syncthreads();
    }
    if (AGG) {
      // the range's end state from zero and its decay exponent
      const int64_t slot = blk.range * (p.nblocks / p.nranges) + bh;
#pragma unroll
      for (int k = 0; k < NTL; ++k)
        *reinterpret_cast<float4*>(p.agg_S + (slot * kP + pp) * N + tile_n0(k)) =
            make_float4(st[k][0], st[k][1], st[k][2], st[k][3]);
      if (tid == 0) p.agg_cs[slot] = cs_sum;
    } else {
      float* const fin = rev ? p.g_first : p.h_last;
      if (fin && blk.range == p.nranges - 1) {
#pragma unroll
        for (int k = 0; k < NTL; ++k)
          *reinterpret_cast<float4*>(fin + ((b * p.H + h) * kP + pp) * N + tile_n0(k)) =
              make_float4(st[k][0], st[k][1], st[k][2], st[k][3]);
      }
    }
  } else {
    // ================= staging waves =================
    // Waves 0..2 of them form the causal C B^T blocks; waves 2, 3 load and
    // commit the chunks' tiles, the last also forms the decays. (The compute
    // waves store the output, so no wave that waits for loads has stores
    // outstanding: stores count in the same wait counter.)
    const int sw = wave - kMainBf;                 // staging wave 0 .. kStageBf-1
    const bool loader = sw >= 2;
    const int lt = tid - 64 * (kMainBf + 2);       // loading thread 0 .. 127
    const int mtb = sw == 0 ? 0 : 1, msb = sw == 2 ? 1 : 0;  // causal C B^T block of staging waves 0..2

    // causal block of C B^T of chunk buffer buf, masked and decayed: M[t][s]
    // = (C_t . B_s) e^{cs_t - cs_s} dt_s, s <= t, as the block of B C^T:
    // register r of the lane is s = 16 msb + 4 lk + r, t = 16 mtb + li
    auto causal_block = [&](const int buf) {
      uint4 bb[KN], cc[KN];
#pragma unroll
      for (int j = 0; j < KN; ++j) {
        bb[j] = *reinterpret_cast<const uint4*>(&sm.B[buf][16 * msb + li][32 * j + 8 * lk]);
        cc[j] = *reinterpret_cast<const uint4*>(&sm.C[buf][16 * mtb + li][32 * j + 8 * lk]);
      }
      f4 a = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int j = 0; j < KN; ++j) a = mfma_bf16(bb[j], cc[j], a);
      const int t = 16 * mtb + li, s0 = 16 * msb + 4 * lk;
      const float cst = sm.cs[buf][t];
      const float4 css = *reinterpret_cast<const float4*>(&sm.cs[buf][s0]);
      const float4 dts = *reinterpret_cast<const float4*>(&sm.dt[buf][s0]);
      const float m0 = s0 + 0 <= t ? a[0] * __expf(cst - css.x) * dts.x : 0.f;
      const float m1 = s0 + 1 <= t ? a[1] * __expf(cst - css.y) * dts.y : 0.f;
      const float m2 = s0 + 2 <= t ? a[2] * __expf(cst - css.z) * dts.z : 0.f;
      const float m3 = s0 + 3 <= t ? a[3] * __expf(cst - css.w) * dts.w : 0.f;
      uint32_t h01, l01, h23, l23;
      split_pack_bf16(m0, m1, h01, l01);
      split_pack_bf16(m2, m3, h23, l23);
      *reinterpret_cast<uint2*>(&sm.M[buf][0][t][s0]) = make_uint2(h01, h23);
      *reinterpret_cast<uint2*>(&sm.M[buf][1][t][s0]) = make_uint2(l01, l23);
    };

    if (loader) {
      // one stager: the next chunk's tiles are loaded during phase 1 and
      // committed in phase 2 of the same chunk (with two stagers a chunk
      // ahead the compiler's waits took in the newest loads as well)
      SsdStagerBf<N, 128> stg;
      stg.init(p, lt, b, h, g, c0 * kQ, rev);
      stg.load(p, lt, c0 * kQ);
      stg.commit(p, bias, sm, 0, lt);
      if (sw == kStageBf - 1) chunk_decay(sm, 0, Ah, lane, stg.dt_value(p, bias));
      __syncthreads();
      for (int64_t c = c0; c < c1; ++c) {
        const int cur = (c - c0) & 1, nxt = cur ^ 1;
        // ---- phase 1: the chunk's M; the loads of the next chunk ----
        if (!AGG && sw == 2) causal_block(cur);
        if (c + 1 < c1) stg.load(p, lt, (c + 1) * kQ);
        __syncthreads();
        // ---- phase 2: the next chunk's tiles and decays ----
        if (c + 1 < c1) {
          stg.commit(p, bias, sm, nxt, lt);
          if (sw == kStageBf - 1) chunk_decay(sm, nxt, Ah, lane, stg.dt_value(p, bias));
        }
        __syncthreads();
      }
    } else {
      __syncthreads();
      for (int64_t c = c0; c < c1; ++c) {
        const int cur = (c - c0) & 1;
        // ---- phase 1: the chunk's M ----
        if (!AGG) causal_block(cur);
        __syncthreads();
        __syncthreads();
      }
    }
  }
}

template <int N, bool BIDIR, bool GATE, bool AGG = false>
__global__ __launch_bounds__(64 * kWavesBf) void ssd_fwd_bf16_kernel(const SsdArgs<uint16_t> p) {
  static_assert(kQ == 32 && kP == 64 && kMainBf == 8 && kStageBf == 4, "work split below assumes these sizes");
  static_assert(N == 64 || N == 128, "state sizes");
  static_assert(!(AGG && (BIDIR || GATE)), "the aggregate pass runs one sweep, no gate");

  __shared__ SsdSmemBf<N> sm;

  const SsdBlock blk = ssd_block(p);
  const int64_t h = blk.bh % p.H;
  const float Dfwd = p.D ? p.D[h] : 0.f;
  const float bias = p.dt_bias ? p.dt_bias[h] : 0.f;  // the head's step-size bias (0: none), in a register

  // the block t < 16, s >= 16 of M stays zero (future steps)
  for (int i = threadIdx.x; i < 4 * kQ * SsdSmemBf<N>::TP; i += 64 * kWavesBf) (&sm.M[0][0][0][0])[i] = 0;

  // BIDIR: a reverse sweep (zero initial state, no D x) storing a float32
  // partial, then the forward sweep adding it (a split sequence runs them in
  // separate launches: sweep_sel). Without BIDIR, sweep_sel 0 selects the
  // reverse sweep: only the aggregate pass of a split bidirectional scan
  // runs that way.
  if (BIDIR) {
    if (p.sweep_sel != 1) {
      ssd_bf16_sweep<N, BIDIR, GATE, AGG, true>(p, sm, blk, Dfwd, bias);
      // the forward sweep reuses the LDS tiles and reads the partial just stored
      __syncthreads();
    }
    if (p.sweep_sel != 0) ssd_bf16_sweep<N, BIDIR, GATE, AGG, false>(p, sm, blk, Dfwd, bias);
  } else if (AGG && p.sweep_sel == 0) {
    ssd_bf16_sweep<N, BIDIR, GATE, AGG, true>(p, sm, blk, Dfwd, bias);
  } else {
    ssd_bf16_sweep<N, BIDIR, GATE, AGG, false>(p, sm, blk, Dfwd, bias);
  }
}

int ssd_validate(const void* x, const void* dt, const float* A, const void* B, const void* C, const float* D,
                 const float* h0, const float* g0, const ssm_scan_options* opts, const void* y, const float* h_last,
                 const float* g_first, int64_t Bs, int64_t L, int64_t H, int64_t P, int64_t G, int64_t N,
                 int dtype) {
  // Bs and L may be zero (empty tensors); H, P, G and N are positive
  if (Bs < 0 || L < 0 || H <= 0 || P <= 0 || G <= 0 || N <= 0) return SSM_ERR_DIM;
  int64_t t, rows, seq, bc, state, hd;
  if (!mul_nn(Bs, L, &rows) || !mul_nn(rows, H, &hd) || !mul_nn(hd, P, &seq) || !mul_nn(rows, G, &t) ||
      !mul_nn(t, N, &bc) || !mul_nn(Bs, H, &t) || !mul_nn(t, P, &t) || !mul_nn(t, N, &state))
    return SSM_ERR_DIM;
  // a buffer with no elements may be NULL
  if (!A || (seq > 0 && (!x || !dt || !y || !B || !C))) return SSM_ERR_NULL;
  if (seq > INT64_MAX / 8 || bc > INT64_MAX / 8 || state > INT64_MAX / 8) return SSM_ERR_DIM;
  if (H % G != 0) return SSM_ERR_DIM;
  if (dtype != SSM_F32 && dtype != SSM_BF16) return SSM_ERR_UNSUPPORTED;
  if (P != kP || (N != 64 && N != 128)) return SSM_ERR_UNSUPPORTED;
  if (Bs * H > INT32_MAX || L >= (int64_t{1} << 36)) return SSM_ERR_DIM;
  const float* dt_bias = opts ? opts->dt_bias : nullptr;
  const void* z = opts ? opts->z : nullptr;
  if (opts && !(opts->dt_min <= opts->dt_max)) return SSM_ERR_ARG;  // also catches NaN
  const void* ptrs[] = {x, dt, A, B, C, D, h0, g0, dt_bias, z, y, h_last, g_first};
  for (const void* q : ptrs)
    if (q && !aligned16(q)) return SSM_ERR_UNSUPPORTED;
  const int64_t es = dtype == SSM_F32 ? 4 : 2;
  const Range in[] = {rng(x, seq * es), rng(dt, hd * es), rng(A, H * 4), rng(B, bc * es), rng(C, bc * es),
                      rng(D, D ? H * 4 : 0), rng(h0, h0 ? state * 4 : 0), rng(g0, g0 ? state * 4 : 0),
                      rng(dt_bias, dt_bias ? H * 4 : 0), rng(z, z ? seq * es : 0)};
  const Range out[] = {rng(y, seq * es), rng(h_last, h_last ? state * 4 : 0), rng(g_first, g_first ? state * 4 : 0)};
  for (int i = 0; i < 3; ++i) {
    if (out[i].hi == out[i].lo) continue;
    for (const Range& r : in)
      if (r.hi > r.lo && overlap(out[i], r)) return SSM_ERR_ALIAS;
    for (int j = 0; j < i; ++j)
      if (out[j].hi > out[j].lo && overlap(out[i], out[j])) return SSM_ERR_ALIAS;
  }
  return SSM_OK;
}

// float32 partial of the bidirectional scan's reverse sweep: into y for
// float32, into the workspace for bf16. Another wave of the same workgroup
// reads each value in the forward sweep; the workgroup barrier that ends the
// reverse sweep orders the stores before those loads.
// How a multi-head scan splits its sequences: one workgroup per (batch row,
// head) holds a compute unit (its LDS), so with fewer pairs than CUs each
// sweep is cut into ranges of whole chunks (at least 8 chunks each), about one
// workgroup per CU in all. A first pass (the AGG kernels) forms every range's
// end state from zero and its decay exponent; the second runs every range
// from the state folded in from the ranges before it. Nothing waits on
// another workgroup.
struct SsdPlan {
  int64_t nranges, range_chunks;
  size_t agg_bytes;  // per sweep: end states (sized for N = 128) and decay exponents
};

SsdPlan ssd_plan(int64_t Bs, int64_t L, int64_t H) {
  SsdPlan sp{};
  const int64_t nbh = Bs * H, nchunks = (L + kQ - 1) / kQ, ncu = device_cus();
  sp.nranges = 1;
  sp.range_chunks = nchunks;
  if (ncu > 0 && nbh > 0 && nbh < ncu) {
    const int64_t k = std::min<int64_t>(ncu / nbh, nchunks / 8);
    if (k >= 2) {
      sp.range_chunks = (nchunks + k - 1) / k;
      sp.nranges = (nchunks + sp.range_chunks - 1) / sp.range_chunks;
    }
  }
  if (sp.nranges > 1) {
    const size_t slots = static_cast<size_t>(nbh * sp.nranges);
    sp.agg_bytes = ((slots * kP * 128 * 4 + 255) & ~static_cast<size_t>(255)) + ((slots * 8 + 255) & ~static_cast<size_t>(255));
  }
  return sp;
}

// workspace: [float32 partials of the bidirectional bf16 scan] [split plan:
// the forward sweep's aggregates] [the reverse sweep's aggregates]
size_t ssd_partial_bytes(int64_t Bs, int64_t L, int64_t H, int64_t P, int dtype, bool bidir) {
  if (!bidir || dtype != SSM_BF16) return 0;
  int64_t n;
  if (!mul_ok(Bs, L, &n) || !mul_ok(n, H, &n) || !mul_ok(n, P, &n) || n > INT64_MAX / 8) return 0;
  return (static_cast<size_t>(n) * 4 + 255) & ~static_cast<size_t>(255);
}

size_t ssd_ws_bytes(int64_t Bs, int64_t L, int64_t H, int64_t P, int dtype, bool bidir) {
  if (Bs <= 0 || L <= 0 || H <= 0 || P <= 0 || Bs * H > INT32_MAX / 64) return 0;
  if (dtype != SSM_F32 && dtype != SSM_BF16) return 0;
  const SsdPlan sp = ssd_plan(Bs, L, H);
  return ssd_partial_bytes(Bs, L, H, P, dtype, bidir) + (bidir ? 2 : 1) * sp.agg_bytes;
}

template <typename T, bool BIDIR, bool GATE, bool AGG = false>
void launch_ssd_kernel(const SsdArgs<T>& a, int64_t N, dim3 grid, dim3 block, hipStream_t stream) {
  if constexpr (std::is_same<T, uint16_t>::value) {
    const dim3 bblock(64 * kWavesBf);
    if (N == 128) hipLaunchKernelGGL((ssd_fwd_bf16_kernel<128, BIDIR, GATE, AGG>), grid, bblock, 0, stream, a);
    else hipLaunchKernelGGL((ssd_fwd_bf16_kernel<64, BIDIR, GATE, AGG>), grid, bblock, 0, stream, a);
  } else {
    if (N == 128) hipLaunchKernelGGL((ssd_fwd_kernel<T, 128, BIDIR, GATE, AGG>), grid, block, 0, stream, a);
    else hipLaunchKernelGGL((ssd_fwd_kernel<T, 64, BIDIR, GATE, AGG>), grid, block, 0, stream, a);
  }
}

template <typename T>
int launch_ssd(const void* x, const void* dt, const float* A, const void* B, const void* C, const float* D,
               const float* h0, const float* g0, const ssm_scan_options* opts, void* y, float* h_last, float* g_first, float* part,
               bool bidir, int64_t Bs, int64_t L, int64_t H, int64_t G, int64_t N, void* ws, hipStream_t stream) {
  SsdArgs<T> a;
  a.x = static_cast<const T*>(x);
  a.dt = static_cast<const T*>(dt);
  a.A = A;
  a.B = static_cast<const T*>(B);
  a.C = static_cast<const T*>(C);
  a.D = D;
  a.h0 = h0;
  a.g0 = bidir ? g0 : nullptr;
  a.y = static_cast<T*>(y);
  a.h_last = h_last;
  a.part = part;
  a.g_first = g_first;
  a.dt_bias = opts ? opts->dt_bias : nullptr;
  a.dt_softplus = opts && opts->dt_softplus ? 1 : 0;
  a.dt_min = opts ? opts->dt_min : -INFINITY;
  a.dt_max = opts ? opts->dt_max : INFINITY;
  a.dt_pre = (a.dt_bias || a.dt_softplus || a.dt_min > -INFINITY || a.dt_max < INFINITY) ? 1 : 0;
  a.z = opts ? static_cast<const T*>(opts->z) : nullptr;
  a.L = L;
  a.H = H;
  a.G = G;
  const SsdPlan sp = ssd_plan(Bs, L, H);
  a.nranges = static_cast<int>(sp.nranges);
  a.range_chunks = sp.range_chunks;
  a.sweep_sel = -1;
  a.agg_S = nullptr;
  a.agg_cs = nullptr;
  a.nblocks = static_cast<int>(Bs * H * sp.nranges);
  const dim3 grid(static_cast<unsigned>(a.nblocks)), block(64 * kWaves);
  if (sp.nranges > 1) {
    // the sweeps' aggregates (forward, then reverse), then every range from
    // its folded entering state; the bidirectional scan stores the reverse
    // sweep's partials in a launch of their own before the forward sweep
    // reads them
    const size_t slots = static_cast<size_t>(Bs * H * sp.nranges);
    const size_t s_bytes = (slots * kP * 128 * 4 + 255) & ~static_cast<size_t>(255);
    char* w = static_cast<char*>(ws) + ssd_partial_bytes(Bs, L, H, kP, std::is_same<T, float>::value ? SSM_F32 : SSM_BF16, bidir);
    const int64_t nbh = Bs * H, PN = kP * N;
    const dim3 jgrid(static_cast<unsigned>((nbh * PN + 255) / 256)), jblock(256);
    SsdArgs<T> fw = a, rv = a;
    fw.agg_S = reinterpret_cast<float*>(w);
    fw.agg_cs = reinterpret_cast<double*>(w + s_bytes);
    fw.sweep_sel = 1;
    launch_ssd_kernel<T, false, false, true>(fw, N, grid, block, stream);
    hipLaunchKernelGGL(ssd_join_kernel, jgrid, jblock, 0, stream, fw.agg_S, fw.agg_cs, h0, nbh, sp.nranges, PN);
    if (bidir) {
      rv.agg_S = reinterpret_cast<float*>(w + sp.agg_bytes);
      rv.agg_cs = reinterpret_cast<double*>(w + sp.agg_bytes + s_bytes);
      rv.sweep_sel = 0;
      launch_ssd_kernel<T, false, false, true>(rv, N, grid, block, stream);
      hipLaunchKernelGGL(ssd_join_kernel, jgrid, jblock, 0, stream, rv.agg_S, rv.agg_cs, g0, nbh, sp.nranges, PN);
      if (rv.z) launch_ssd_kernel<T, true, true>(rv, N, grid, block, stream);
      else launch_ssd_kernel<T, true, false>(rv, N, grid, block, stream);
      if (fw.z) launch_ssd_kernel<T, true, true>(fw, N, grid, block, stream);
      else launch_ssd_kernel<T, true, false>(fw, N, grid, block, stream);
    } else {
      if (fw.z) launch_ssd_kernel<T, false, true>(fw, N, grid, block, stream);
      else launch_ssd_kernel<T, false, false>(fw, N, grid, block, stream);
    }
    return hipGetLastError() == hipSuccess ? SSM_OK : SSM_ERR_LAUNCH;
  }
  if (bidir) {
    if (a.z) launch_ssd_kernel<T, true, true>(a, N, grid, block, stream);
    else launch_ssd_kernel<T, true, false>(a, N, grid, block, stream);
  } else {
    if (a.z) launch_ssd_kernel<T, false, true>(a, N, grid, block, stream);
    else launch_ssd_kernel<T, false, false>(a, N, grid, block, stream);
  }
  return hipGetLastError() == hipSuccess ? SSM_OK : SSM_ERR_LAUNCH;
}

// An empty batch or sequence: nothing to scan. Over zero steps each state
// stays where it entered (h_last = h0, g_first = g0, or zero).
int ssd_empty(const float* h0, const float* g0, float* h_last, float* g_first, int64_t state, hipStream_t stream) {
  const bool ok = fill_async(h_last, h0, state * 4, stream) && fill_async(g_first, g0, state * 4, stream);
  return ok ? SSM_OK : SSM_ERR_LAUNCH;
}

// The workspace may not overlap any argument.
int ssd_check_workspace(const void* x, const void* dt, const float* A, const void* B, const void* C, const float* D,
                        const float* h0, const float* g0, const ssm_scan_options* opts, const void* y,
                        const float* h_last, const float* g_first, int64_t Bs, int64_t L, int64_t H, int64_t P,
                        int64_t G, int64_t N, int dtype, const void* workspace, size_t workspace_bytes, size_t need) {
  if (need == 0) return SSM_OK;
  if (!workspace || workspace_bytes < need || !aligned16(workspace)) return SSM_ERR_WORKSPACE;
  const int64_t es = dtype == SSM_F32 ? 4 : 2;
  const int64_t seq = Bs * L * H * P, hd = Bs * L * H, bc = Bs * L * G * N, state = Bs * H * P * N;
  const Range ws = rng(workspace, static_cast<int64_t>(need));
  const float* dt_bias = opts ? opts->dt_bias : nullptr;
  const void* z = opts ? opts->z : nullptr;
  const Range args[] = {rng(x, seq * es), rng(dt, hd * es), rng(A, H * 4), rng(B, bc * es), rng(C, bc * es),
                        rng(D, D ? H * 4 : 0), rng(h0, h0 ? state * 4 : 0), rng(g0, g0 ? state * 4 : 0),
                        rng(y, seq * es),
                        rng(h_last, h_last ? state * 4 : 0), rng(g_first, g_first ? state * 4 : 0),
                        rng(dt_bias, dt_bias ? H * 4 : 0), rng(z, z ? seq * es : 0)};
  for (const Range& r : args)
    if (r.hi > r.lo && overlap(ws, r)) return SSM_ERR_ALIAS;
  return SSM_OK;
}

}  // namespace

extern "C" size_t ssm_ssd_workspace_bytes(int64_t Bs, int64_t L, int64_t H, int64_t P, int dtype) {
  return ssd_ws_bytes(Bs, L, H, P, dtype, false);
}

extern "C" int ssm_ssd_fwd(const void* x, const void* dt, const float* A, const void* B, const void* C,
                           const float* D, const float* h0, const ssm_scan_options* opts, void* y, float* h_last,
                           int64_t Bs, int64_t L, int64_t H, int64_t P, int64_t G, int64_t N, int dtype,
                           void* workspace, size_t workspace_bytes, void* stream) {
  int rc = ssd_validate(x, dt, A, B, C, D, h0, nullptr, opts, y, h_last, nullptr, Bs, L, H, P, G, N, dtype);
  if (rc != SSM_OK) return rc;
  hipStream_t st = static_cast<hipStream_t>(stream);
  if (Bs == 0 || L == 0) return ssd_empty(h0, nullptr, h_last, nullptr, Bs * H * P * N, st);
  rc = ssd_check_workspace(x, dt, A, B, C, D, h0, nullptr, opts, y, h_last, nullptr, Bs, L, H, P, G, N, dtype,
                           workspace, workspace_bytes, ssd_ws_bytes(Bs, L, H, P, dtype, false));
  if (rc != SSM_OK) return rc;
  if (dtype == SSM_F32)
    return launch_ssd<float>(x, dt, A, B, C, D, h0, nullptr, opts, y, h_last, nullptr, nullptr, false, Bs, L, H, G, N,
                             workspace, st);
  return launch_ssd<uint16_t>(x, dt, A, B, C, D, h0, nullptr, opts, y, h_last, nullptr, nullptr, false, Bs, L, H, G,
                              N, workspace, st);
}

extern "C" size_t ssm_ssd_bidir_workspace_bytes(int64_t Bs, int64_t L, int64_t H, int64_t P, int dtype) {
  return ssd_ws_bytes(Bs, L, H, P, dtype, true);
}

extern "C" int ssm_ssd_bidir_fwd(const void* x, const void* dt, const float* A, const void* B, const void* C,
                                 const float* D, const float* h0, const float* g0, const ssm_scan_options* opts,
                                 void* y, float* h_last, float* g_first, int64_t Bs, int64_t L, int64_t H, int64_t P,
                                 int64_t G, int64_t N, int dtype, void* workspace, size_t workspace_bytes,
                                 void* stream) {
  int rc = ssd_validate(x, dt, A, B, C, D, h0, g0, opts, y, h_last, g_first, Bs, L, H, P, G, N, dtype);
  if (rc != SSM_OK) return rc;
  hipStream_t st = static_cast<hipStream_t>(stream);
  if (Bs == 0 || L == 0) return ssd_empty(h0, g0, h_last, g_first, Bs * H * P * N, st);
  rc = ssd_check_workspace(x, dt, A, B, C, D, h0, g0, opts, y, h_last, g_first, Bs, L, H, P, G, N, dtype, workspace,
                           workspace_bytes, ssd_ws_bytes(Bs, L, H, P, dtype, true));
  if (rc != SSM_OK) return rc;
  if (dtype == SSM_F32)
    return launch_ssd<float>(x, dt, A, B, C, D, h0, g0, opts, y, h_last, g_first, static_cast<float*>(y), true, Bs, L,
                             H, G, N, workspace, st);
  return launch_ssd<uint16_t>(x, dt, A, B, C, D, h0, g0, opts, y, h_last, g_first, static_cast<float*>(workspace),
                              true, Bs, L, H, G, N, workspace, st);
}
