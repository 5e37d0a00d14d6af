// Backward pass of the selective scan for MI355X (gfx950).
//
// Given dy = dL/dy for the forward scan
//   a_t = exp(delta_t A[e,n]),  h_t = a_t h_{t-1} + (delta_t x_t) B_t[n],
//   y_t = sum_n C_t[n] h_t[n] + D[e] x_t,          h_{-1} = h0 (or zero),
// it returns every input's gradient. This is the step after the forward in
// the autograd function of "Some questions of Bi-Mamba2 and Hydra" (the
// backward listing: dx, ddt, dA, dB, dC, dD from dout); the pages give no
// formula, so the kernel computes the adjoint of the recurrence. With
// g_t = dL/dh_t and k_t = a_t g_t (the part of g_t that reaches step t-1):
//   g_t = dy_t C_t + k_{t+1},          k_L = 0
//   dx_t     = delta_t sum_n g_t B_t + D dy_t
//   ddelta_t = x_t sum_n g_t B_t + sum_n A g_t a_t h_{t-1}
//   dB_t[n]  = sum_e g_t delta_t x_t      dC_t[n] = sum_e dy_t h_t
//   dA[e,n]  = sum_{b,t} delta_t g_t a_t h_{t-1}
//   dD[e]    = sum_{b,t} dy_t x_t          dh0 = k_0
//
// Work: one workgroup per (batch row, 16 consecutive channels), the lane
// layout of the forward kernel (lane = 16 r + 4 g + c holds channel 4 r + c
// and states 4 g .. 4 g + 3), SEG waves, each owning TS consecutive steps of
// a round of RT = SEG * TS steps.
//   sweep 1 (increasing rounds): the forward scan's round aggregates only
//     (no per-step replay, no output); the state entering each round is
//     written to a workspace checkpoint.
//   sweep 2 (decreasing rounds): per round, the forward states are rebuilt
//     from the checkpoint (local pass, fold, replay that keeps h_{t-1} of
//     every step in registers), then the adjoint runs backward in time the
//     same way (local pass from a zero carry, fold over the later segments
//     and the next round's carry, replay) and every gradient term of the step
//     is formed in the replay (dx and ddelta go to the round's LDS tile
//     and out one round later, 4 channels per store). Sums over the lane's
//     4 states and over the 4 state quads of a channel go through DPP; sums
//     over the 16 channels of
//     dB and dC go through DPP (over the quad) and LDS (over the 4 lane rows)
//     into per-workgroup partials that a second kernel adds up in a fixed
//     order (no atomics: the result is deterministic).
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <cstdint>
#include <type_traits>

#include "scan_common.h"
#include "ssm_scan.h"

namespace {

constexpr int kBSEG = 4, kBTS = 8, kBRT = kBSEG * kBTS;

template <typename T>
struct BwdArgs {
  const T* x;
  const T* dl;
  const float* A;
  const T* B;
  const T* C;
  const float* D;    // or nullptr
  const float* h0;   // or nullptr
  const float* dh_last;  // gradient of the final state (Bs, ED, N): the adjoint carry entering the last step, or nullptr
  // step-size options of the forward: delta' = clamp(softplus?(delta + dt_bias), dt_min, dt_max)
  const float* dt_bias;  // (ED) or nullptr
  int dt_softplus;
  int dt_pre;            // any option at all
  float dt_min, dt_max;
  double* pDB;       // [Bs][EDp]: ddt_bias partial of each batch row, or nullptr
  const T* dy;
  const float* dyf;  // float32 output gradient read instead of dy (behind the gate; OPTS kernels only), or nullptr
  T* dx;
  T* ddl;
  float* dh0;        // or nullptr
  float* ckpt;       // [Bs][rounds][EDp][16]: state entering each round (round 0 unused)
  int ck_given;      // the caller's checkpoints (of the forward scan): the first sweep is skipped
  float* pB;         // [ngroups][Bs][L][16]: dB partial of each channel group
  float* pC;         // same for dC
  double* pA;        // [Bs][EDp][16]: dA partial of each batch row
  double* pD;        // [Bs][EDp]: dD partial of each batch row
  int64_t Bs, L, ED, EDp, rounds;
  int ngroups;
  int nblocks;
  int remap;
  int rot_ncu;  // compute units, when every workgroup is resident at once; else 0 (no priority rotation)
  // bidirectional backward: the first (forward-time) launch may write dx and
  // ddelta as float32 partials (part_dx, part_dd) instead of the outputs; the
  // second (reverse-time, REV) launch adds float32 partials (acc_dx, acc_dd:
  // those, or the float32 outputs themselves) before its one rounding
  float* part_dx;
  float* part_dd;
  const float* acc_dx;
  const float* acc_dd;
  // split sequence (nchunks > 1): chunk k of a (batch row, channel group)
  // covers the sweep's virtual steps [k chunk_len, (k + 1) chunk_len); the
  // chunk aggregates of bwd_chunk_agg_kernel give the states entering it
  int nchunks;
  int64_t chunk_len;
  double* agg_sd;   // [bg * nchunks + k][16 channels]: sum of delta' over the chunk
  float* agg_h;     // [bg * nchunks + k][16][16]: forward state at the chunk's end, from zero
  float* agg_k;     // [bg * nchunks + k][16][16]: adjoint at the chunk's start, from zero after it
};

template <int RT>
struct alignas(16) BwdTile {
  float dt[RT][16];  // delta per channel
  float xv[RT][16];  // x per channel
  float dy[RT][16];  // dL/dy per channel
  float2 bc[RT][16]; // (B_t[q], C_t[q])
};

template <int RT>
struct alignas(16) ColSums {
  float v[RT][4][2][16];  // [step][lane row r][dB, dC][state]: sums over the row's 4 channels
};

template <int SEG>
struct alignas(16) BwdFold {
  float4 A[SEG][64];   // prod of a over each segment
  float4 H[SEG][64];   // forward: segment end state from zero
  float4 K[SEG][64];   // adjoint: k at the segment start from a zero carry
  float4 kc[2][64];    // adjoint carry between rounds, by round parity
};

// The reductions below issue their DPP adds themselves: written as a DPP move
// plus an add, the compiler keeps the move separate when the add is fused
// with a product or sunk into a branch. A DPP read of a VGPR needs two wait
// states after a VALU write of it; each block opens with s_nop 1 for the
// values written before it, and its own writes are read at least two
// instructions later.

// v[i] <- sum of v[i] over the 4 lanes of the quad (lanes c = 0..3: the 4
// channels of a quad that hold the same states)
__device__ __forceinline__ void quad_sum8(float (&v)[8]) {
  asm("s_nop 1\n\t"
#define SSM_QA(I, P) "v_add_f32_dpp %" #I ", %" #I ", %" #I " quad_perm:" P " row_mask:0xf bank_mask:0xf bound_ctrl:1\n\t"
      SSM_QA(0, "[1,0,3,2]") SSM_QA(1, "[1,0,3,2]") SSM_QA(2, "[1,0,3,2]") SSM_QA(3, "[1,0,3,2]")
      SSM_QA(4, "[1,0,3,2]") SSM_QA(5, "[1,0,3,2]") SSM_QA(6, "[1,0,3,2]") SSM_QA(7, "[1,0,3,2]")
      SSM_QA(0, "[2,3,0,1]") SSM_QA(1, "[2,3,0,1]") SSM_QA(2, "[2,3,0,1]") SSM_QA(3, "[2,3,0,1]")
      SSM_QA(4, "[2,3,0,1]") SSM_QA(5, "[2,3,0,1]") SSM_QA(6, "[2,3,0,1]") SSM_QA(7, "[2,3,0,1]")
#undef SSM_QA
      : "+v"(v[0]), "+v"(v[1]), "+v"(v[2]), "+v"(v[3]), "+v"(v[4]), "+v"(v[5]), "+v"(v[6]), "+v"(v[7]));
}

// a, b <- sums over the lanes 4 apart in a row (the 4 state quads of a channel)
__device__ __forceinline__ void bank_sum2(float& a, float& b) {
  asm("s_nop 1\n\t"
      "v_add_f32_dpp %0, %0, %0 row_ror:4 row_mask:0xf bank_mask:0xf bound_ctrl:1\n\t"
      "v_add_f32_dpp %1, %1, %1 row_ror:4 row_mask:0xf bank_mask:0xf bound_ctrl:1\n\t"
      "s_nop 0\n\t"
      "v_add_f32_dpp %0, %0, %0 row_ror:8 row_mask:0xf bank_mask:0xf bound_ctrl:1\n\t"
      "v_add_f32_dpp %1, %1, %1 row_ror:8 row_mask:0xf bank_mask:0xf bound_ctrl:1"
      : "+v"(a), "+v"(b));
}

// g[j] <- g[j] + C_t[4 g + j] dy for j = 0..3 (C_t[q] in lane q of the row)
__device__ __forceinline__ void add_c_dy(float (&gv)[4], float cq, float dyv) {
  asm("s_nop 1\n\t"
      "v_fmac_f32_dpp %0, %4, %5 quad_perm:[0,0,0,0] row_mask:0xf bank_mask:0xf bound_ctrl:1\n\t"
      "v_fmac_f32_dpp %1, %4, %5 quad_perm:[1,1,1,1] row_mask:0xf bank_mask:0xf bound_ctrl:1\n\t"
      "v_fmac_f32_dpp %2, %4, %5 quad_perm:[2,2,2,2] row_mask:0xf bank_mask:0xf bound_ctrl:1\n\t"
      "v_fmac_f32_dpp %3, %4, %5 quad_perm:[3,3,3,3] row_mask:0xf bank_mask:0xf bound_ctrl:1"
      : "+v"(gv[0]), "+v"(gv[1]), "+v"(gv[2]), "+v"(gv[3])
      : "v"(cq), "v"(dyv));
}

// Staging: one task per thread. Threads 0 .. 4 RT - 1 own a (row, 4-channel
// chunk) of x / delta / dy, the others a (row, 4-state chunk) of B / C.
// REV: the reverse-time scan of the bidirectional form. Virtual step t of the
// sweeps is time L - 1 - t: every load and store maps the time, nothing else
// changes (the inputs are read in place, no flipped copy).
// OPTS: the forward ran with step-size options (delta' = the map of delta);
// these kernels also take the output gradient in float32 (dyf) when it is set.
template <typename T, int RT, bool VEC, bool REV, bool OPTS>
struct BwdStager {
  int row, chk;
  bool is_xd, chunk_ok, row_ok;
  float4 ra, rb, rc;
  float4 bias4;  // OPTS: dt_bias of the task's channels
  int64_t b, e0, ED, L;
  int64_t tv0, tv1;  // the virtual steps [tv0, tv1) of this workgroup's chunk (the whole sweep unless split)
  // this task's raw step-size gradients, summed over its rounds in float64
  // (a float32 sum over thousands of rounds would lose the small terms)
  double dbacc[4] = {0.0, 0.0, 0.0, 0.0};

  __device__ __forceinline__ void init(int tid, int64_t b_, int64_t e0_, int64_t ED_, int64_t L_, int64_t tv0_,
                                       int64_t tv1_) {
    int u = tid;
    is_xd = u < 4 * RT;
    if (!is_xd) u -= 4 * RT;
    row = u >> 2;
    chk = u & 3;
    b = b_, e0 = e0_, ED = ED_, L = L_;
    tv0 = tv0_, tv1 = tv1_;
    chunk_ok = !is_xd || e0 + 4 * chk < ED;
  }

  // global -> registers for round rr of the chunk; WITH_ADJ also loads dy and
  // C; without WITH_FWD, x and B are not loaded (their slots hold zeros)
  template <bool WITH_ADJ, bool WITH_FWD = true>
  __device__ __forceinline__ void prefetch(const BwdArgs<T>& p, int64_t rr) {
    const int64_t tv = tv0 + rr * RT + row;
    row_ok = tv < tv1;
    const int64_t t = REV ? L - 1 - tv : tv;
    float4 a = make_float4(0.f, 0.f, 0.f, 0.f), bb = a, cc = a;
    if (row_ok && chunk_ok) {
      if (!is_xd) {
        const int64_t off = (b * L + t) * 16 + 4 * chk;
        if (WITH_FWD) a = Vec4<T>::load(p.B + off);
        if (WITH_ADJ) bb = Vec4<T>::load(p.C + off);
      } else {
        const int64_t ce = e0 + 4 * chk;
        const int64_t off = (b * L + t) * ED + ce;
        if (VEC) {
          if (WITH_FWD) a = Vec4<T>::load(p.x + off);
          bb = Vec4<T>::load(p.dl + off);
          if (WITH_ADJ) cc = (OPTS && p.dyf) ? Vec4<float>::load(p.dyf + off) : Vec4<T>::load(p.dy + off);
        } else {
          if (WITH_FWD)
            a = make_float4(to_f32(p.x[off]), ce + 1 < ED ? to_f32(p.x[off + 1]) : 0.f,
                            ce + 2 < ED ? to_f32(p.x[off + 2]) : 0.f, ce + 3 < ED ? to_f32(p.x[off + 3]) : 0.f);
          bb = make_float4(to_f32(p.dl[off]), ce + 1 < ED ? to_f32(p.dl[off + 1]) : 0.f,
                           ce + 2 < ED ? to_f32(p.dl[off + 2]) : 0.f, ce + 3 < ED ? to_f32(p.dl[off + 3]) : 0.f);
          if (WITH_ADJ && OPTS && p.dyf)
            cc = make_float4(p.dyf[off], ce + 1 < ED ? p.dyf[off + 1] : 0.f, ce + 2 < ED ? p.dyf[off + 2] : 0.f,
                             ce + 3 < ED ? p.dyf[off + 3] : 0.f);
          else if (WITH_ADJ)
            cc = make_float4(to_f32(p.dy[off]), ce + 1 < ED ? to_f32(p.dy[off + 1]) : 0.f,
                             ce + 2 < ED ? to_f32(p.dy[off + 2]) : 0.f, ce + 3 < ED ? to_f32(p.dy[off + 3]) : 0.f);
        }
      }
    }
    ra = a, rb = bb, rc = cc;
  }

  // dx and ddelta of round rr (written into the x and dy slots of its tile by
  // the adjoint replay) -> global
  // d delta'/d delta from delta' itself: 0 where the clamp holds it at a bound,
  // else the softplus derivative sigmoid(v) = 1 - exp(-softplus(v)) (or 1)
  // OPTS: the biases of the thread's 4 channels, loaded once (the channels
  // of a staging task do not change between rounds)
  __device__ __forceinline__ void load_bias(const BwdArgs<T>& p) {
    bias4 = make_float4(0.f, 0.f, 0.f, 0.f);
    if (!OPTS || !p.dt_bias || !is_xd || !chunk_ok) return;
    const int64_t ce = e0 + 4 * chk;
    bias4 = make_float4(p.dt_bias[ce], ce + 1 < ED ? p.dt_bias[ce + 1] : 0.f, ce + 2 < ED ? p.dt_bias[ce + 2] : 0.f,
                        ce + 3 < ED ? p.dt_bias[ce + 3] : 0.f);
  }

  __device__ __forceinline__ float map_deriv(const BwdArgs<T>& p, float m) const {
    if (m <= p.dt_min || m >= p.dt_max) return 0.f;
    return p.dt_softplus ? -expm1_fast(-m) : 1.f;
  }

  __device__ __forceinline__ void store_grads(const BwdArgs<T>& p, const BwdTile<RT>& tl, int64_t rr) {
    const int64_t tv = tv0 + rr * RT + row;
    if (!is_xd || tv >= tv1 || !chunk_ok) return;
    const int64_t t = REV ? L - 1 - tv : tv;
    const int c4 = 4 * chk;
    float4 gx = *reinterpret_cast<const float4*>(&tl.xv[row][c4]);
    float4 gd = *reinterpret_cast<const float4*>(&tl.dy[row][c4]);
    if constexpr (OPTS) {
      // through the step-size map to the raw step size; ddt_bias sums it
      const float4 m = *reinterpret_cast<const float4*>(&tl.dt[row][c4]);
      gd = make_float4(gd.x * map_deriv(p, m.x), gd.y * map_deriv(p, m.y), gd.z * map_deriv(p, m.z),
                       gd.w * map_deriv(p, m.w));
      dbacc[0] += static_cast<double>(gd.x);
      dbacc[1] += static_cast<double>(gd.y);
      dbacc[2] += static_cast<double>(gd.z);
      dbacc[3] += static_cast<double>(gd.w);
    }
    const int64_t ce = e0 + c4, off = (b * L + t) * ED + ce;
    if (VEC) {
      if (REV && p.acc_dx) {
        const float4 ax = *reinterpret_cast<const float4*>(p.acc_dx + off);
        const float4 ad = *reinterpret_cast<const float4*>(p.acc_dd + off);
        gx = make_float4(gx.x + ax.x, gx.y + ax.y, gx.z + ax.z, gx.w + ax.w);
        gd = make_float4(gd.x + ad.x, gd.y + ad.y, gd.z + ad.z, gd.w + ad.w);
      }
      if (p.part_dx) {
        *reinterpret_cast<float4*>(p.part_dx + off) = gx;
        *reinterpret_cast<float4*>(p.part_dd + off) = gd;
      } else {
        Vec4<T>::store(p.dx + off, gx);
        Vec4<T>::store(p.ddl + off, gd);
      }
    } else {
      float vx[4] = {gx.x, gx.y, gx.z, gx.w}, vd[4] = {gd.x, gd.y, gd.z, gd.w};
#pragma unroll
      for (int k = 0; k < 4; ++k)
        if (ce + k < ED) {
          if (REV && p.acc_dx) {
            vx[k] += p.acc_dx[off + k];
            vd[k] += p.acc_dd[off + k];
          }
          if (p.part_dx) {
            p.part_dx[off + k] = vx[k];
            p.part_dd[off + k] = vd[k];
          } else {
            p.dx[off + k] = from_f32<T>(vx[k]);
            p.ddl[off + k] = from_f32<T>(vd[k]);
          }
        }
    }
  }

  // registers -> LDS tile (padded rows and channels are zero: delta = 0
  // gives a = 1 and b = 0, dy = 0 gives no adjoint input). The tile holds
  // the step size after the options, delta'.
  template <bool WITH_ADJ>
  __device__ __forceinline__ void commit(const BwdArgs<T>& p, BwdTile<RT>& tl) const {
    const int c4 = 4 * chk;
    if (is_xd) {
      *reinterpret_cast<float4*>(&tl.xv[row][c4]) = ra;
      float4 dv = rb;
      if constexpr (OPTS) {
        // (the chunk's biases are in registers: bias4, zero without a bias)
        const bool ok = row_ok && chunk_ok;
        const int64_t ce = e0 + c4;
        dv.x = ok && ce + 0 < ED ? map_step(dv.x + bias4.x, nullptr, p.dt_softplus, p.dt_min, p.dt_max) : 0.f;
        dv.y = ok && ce + 1 < ED ? map_step(dv.y + bias4.y, nullptr, p.dt_softplus, p.dt_min, p.dt_max) : 0.f;
        dv.z = ok && ce + 2 < ED ? map_step(dv.z + bias4.z, nullptr, p.dt_softplus, p.dt_min, p.dt_max) : 0.f;
        dv.w = ok && ce + 3 < ED ? map_step(dv.w + bias4.w, nullptr, p.dt_softplus, p.dt_min, p.dt_max) : 0.f;
      }
      *reinterpret_cast<float4*>(&tl.dt[row][c4]) = dv;
      if (WITH_ADJ) *reinterpret_cast<float4*>(&tl.dy[row][c4]) = rc;
    } else {
      *reinterpret_cast<float4*>(&tl.bc[row][c4]) = make_float4(ra.x, rb.x, ra.y, rb.y);
      *reinterpret_cast<float4*>(&tl.bc[row][c4 + 2]) = make_float4(ra.z, rb.z, ra.w, rb.w);
    }
  }
};

// dB / dC partials of round rr (their column sums are in cs) -> workspace
template <typename T, int RT, bool REV>
__device__ __forceinline__ void store_colsums(const BwdArgs<T>& p, const ColSums<RT>& cs, int tid, int64_t b,
                                              int64_t grp, int64_t tv0, int64_t tv1, int64_t rr) {
  const int tt = tid >> 3, qq = (tid >> 2) & 1, n4 = 4 * (tid & 3);
  const int64_t tv = tv0 + rr * RT + tt;
  if (tv >= tv1) return;
  const int64_t t = REV ? p.L - 1 - tv : tv;
  float4 s = *reinterpret_cast<const float4*>(&cs.v[tt][0][qq][n4]);
#pragma unroll
  for (int r = 1; r < 4; ++r) {
    const float4 v = *reinterpret_cast<const float4*>(&cs.v[tt][r][qq][n4]);
    s = make_float4(s.x + v.x, s.y + v.y, s.z + v.z, s.w + v.w);
  }
  float* dst = qq ? p.pC : p.pB;
  *reinterpret_cast<float4*>(dst + ((grp * p.Bs + b) * p.L + t) * 16 + n4) = s;
}

// The states entering chunk kchunk of a split sweep: the forward state
// h (on entry: h0, or zero) folded through chunks 0 .. kchunk-1, and the
// adjoint k (on entry: dh_last, or zero) folded through chunks nchunks-1 down
// to kchunk+1, each as s = exp2(A log2e sum delta') s + s_chunk in chunk order.
// Given the forward scan's checkpoints, the aggregates hold no forward state
// and h is left as it is (the caller takes the checkpoint of the chunk's
// first round instead).
template <typename T>
__device__ void chunk_entry_states(const BwdArgs<T>& p, int64_t bg, int64_t kchunk, int ch, int g,
                                   const float (&A2)[4], float (&h)[4], float (&k)[4]) {
  const int64_t K = p.nchunks;
  auto fold = [&](float (&v)[4], const float* agg, int64_t j) {
    const int64_t slot = bg * K + j;
    const float sdc = static_cast<float>(p.agg_sd[slot * 16 + ch]);
    const float4 a = *reinterpret_cast<const float4*>(agg + slot * 256 + ch * 16 + 4 * g);
    const float av[4] = {a.x, a.y, a.z, a.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) v[i] = __builtin_fmaf(__builtin_amdgcn_exp2f(A2[i] * sdc), v[i], av[i]);
  };
  if (!p.ck_given) {
#pragma unroll 4
    for (int64_t j = 0; j < kchunk; ++j) fold(h, p.agg_h, j);
  }
#pragma unroll 4
  for (int64_t j = K - 1; j > kchunk; --j) fold(k, p.agg_k, j);
}

// First pass of a split sweep: per (batch row, channel group, chunk), the
// chunk's aggregates from zero states: the sum of delta' over its steps
// (float64), the forward state at its end and the adjoint at its start,
// k = sum_t (prod_{s = t0 .. t} a_s) (dy_t C_t) (each a product of a and the
// adjoint's own input, accumulated along the chunk). The second pass
// (scan_bwd_kernel) folds them into the states entering each chunk.
// FWD = false (the forward scan's checkpoints give the forward states): the
// adjoint and the step sums only, without loading x and B.
template <typename T, int SEG, int TS, bool VEC, bool REV, bool OPTS, bool FWD>
__global__ __launch_bounds__(64 * SEG) __attribute__((amdgpu_waves_per_eu(3))) void bwd_chunk_agg_kernel(
    const BwdArgs<T> p) {
  constexpr int RT = SEG * TS;
  static_assert(SEG * 64 == 8 * RT, "one staging task per thread");
  __shared__ BwdTile<RT> tile[2];
  __shared__ BwdFold<SEG> fa;
  __shared__ float sds[SEG][64];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int q = lane & 15;
  const int g = q >> 2;
  const int c = q & 3;
  const int ch = ((lane >> 4) << 2) | c;
  const int64_t L = p.L, ED = p.ED;
  int blk = blockIdx.x;
  if (p.remap) blk = (blk & 7) * (p.nblocks >> 3) + (blk >> 3);
  const int64_t nbg = p.nblocks / p.nchunks;
  const int64_t kchunk = blk / nbg, bg = blk % nbg;
  const int64_t b = bg / p.ngroups;
  const int64_t e0 = (bg % p.ngroups) * 16;
  const int64_t tv0 = kchunk * p.chunk_len;
  const int64_t tv1 = L - tv0 < p.chunk_len ? L : tv0 + p.chunk_len;
  const int64_t R = (tv1 - tv0 + RT - 1) / RT;
  const int64_t e = e0 + ch;
  const int64_t ec = e < ED ? e : ED - 1;
  float A2[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) A2[j] = p.A[ec * 16 + 4 * g + j] * kLog2e;

  BwdStager<T, RT, VEC, REV, OPTS> st;
  st.init(tid, b, e0, ED, L, tv0, tv1);
  st.load_bias(p);
  float hc[4] = {0.f, 0.f, 0.f, 0.f};  // forward state (wave SEG-1)
  float kc[4] = {0.f, 0.f, 0.f, 0.f};  // adjoint at the chunk's start, so far (wave SEG-1)
  double sdc = 0.0;                    // sum of delta' before the current segment (wave SEG-1)
  st.template prefetch<true, FWD>(p, 0);
  st.template commit<true>(p, tile[0]);
  __syncthreads();
  for (int64_t r = 0; r < R; ++r) {
    rotate_priority(r, p.rot_ncu);
    BwdTile<RT>& cur = tile[r & 1];
    BwdTile<RT>& nxt = tile[(r + 1) & 1];
    if (r + 1 < R) st.template prefetch<true, FWD>(p, r + 1);
    // this wave's segment from zero: the forward end state, and the adjoint
    // at the segment's start (backwards over its steps)
    float av[TS][4], hl[4] = {0.f, 0.f, 0.f, 0.f}, kl[4] = {0.f, 0.f, 0.f, 0.f}, sd = 0.f;
#pragma unroll
    for (int i = 0; i < TS; ++i) {
      const int row = wave * TS + i;
      const float dt = cur.dt[row][ch];
      sd += dt;
#pragma unroll
      for (int j = 0; j < 4; ++j) av[i][j] = __builtin_amdgcn_exp2f(dt * A2[j]);
      if constexpr (FWD) {
        const float dxv = dt * cur.xv[row][ch];
        const float bq = cur.bc[row][q].x;
        const float bb[4] = {quad_bcast<0>(bq), quad_bcast<1>(bq), quad_bcast<2>(bq), quad_bcast<3>(bq)};
#pragma unroll
        for (int j = 0; j < 4; ++j) hl[j] = __builtin_fmaf(av[i][j], hl[j], dxv * bb[j]);
      }
    }
#pragma unroll
    for (int i = TS - 1; i >= 0; --i) {
      const int row = wave * TS + i;
      add_c_dy(kl, cur.bc[row][q].y, cur.dy[row][ch]);
#pragma unroll
      for (int j = 0; j < 4; ++j) kl[j] *= av[i][j];
    }
    if constexpr (FWD) {
      fa.A[wave][lane] = make_float4(__builtin_amdgcn_exp2f(A2[0] * sd), __builtin_amdgcn_exp2f(A2[1] * sd),
                                     __builtin_amdgcn_exp2f(A2[2] * sd), __builtin_amdgcn_exp2f(A2[3] * sd));
      fa.H[wave][lane] = make_float4(hl[0], hl[1], hl[2], hl[3]);
    }
    fa.K[wave][lane] = make_float4(kl[0], kl[1], kl[2], kl[3]);
    sds[wave][lane] = sd;
    __syncthreads();
    if (wave == SEG - 1) {
      for (int k = 0; k < SEG; ++k) {
        // the segment's adjoint reaches the chunk's start through every step
        // before it: the product from the float64 sum of delta' so far
        const float cum = static_cast<float>(sdc);
        const float4 Kk = fa.K[k][lane];
        kc[0] = __builtin_fmaf(__builtin_amdgcn_exp2f(A2[0] * cum), Kk.x, kc[0]);
        kc[1] = __builtin_fmaf(__builtin_amdgcn_exp2f(A2[1] * cum), Kk.y, kc[1]);
        kc[2] = __builtin_fmaf(__builtin_amdgcn_exp2f(A2[2] * cum), Kk.z, kc[2]);
        kc[3] = __builtin_fmaf(__builtin_amdgcn_exp2f(A2[3] * cum), Kk.w, kc[3]);
        if constexpr (FWD) {
          const float4 Ak = fa.A[k][lane], Hk = fa.H[k][lane];
          hc[0] = __builtin_fmaf(Ak.x, hc[0], Hk.x);
          hc[1] = __builtin_fmaf(Ak.y, hc[1], Hk.y);
          hc[2] = __builtin_fmaf(Ak.z, hc[2], Hk.z);
          hc[3] = __builtin_fmaf(Ak.w, hc[3], Hk.w);
        }
        sdc += static_cast<double>(sds[k][lane]);
      }
    }
    if (r + 1 < R) st.template commit<true>(p, nxt);
    __syncthreads();
  }
  if (wave == SEG - 1) {
    const int64_t slot = bg * p.nchunks + kchunk;
    if (g == 0) p.agg_sd[slot * 16 + ch] = sdc;
    if (FWD)
      *reinterpret_cast<float4*>(p.agg_h + slot * 256 + ch * 16 + 4 * g) = make_float4(hc[0], hc[1], hc[2], hc[3]);
    *reinterpret_cast<float4*>(p.agg_k + slot * 256 + ch * 16 + 4 * g) = make_float4(kc[0], kc[1], kc[2], kc[3]);
  }
}

template <typename T, int SEG, int TS, bool VEC, bool REV, bool OPTS>
__global__ __launch_bounds__(64 * SEG) __attribute__((amdgpu_waves_per_eu(3))) void scan_bwd_kernel(
    const BwdArgs<T> p) {
  constexpr int RT = SEG * TS;
  static_assert(SEG * 64 == 8 * RT, "one staging task per thread");

  __shared__ BwdTile<RT> tile[2];
  __shared__ ColSums<RT> cs;
  __shared__ BwdFold<SEG> fa;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int q = lane & 15;
  const int g = q >> 2;
  const int c = q & 3;
  const int lrow = lane >> 4;
  const int ch = (lrow << 2) | c;
  const int64_t L = p.L, ED = p.ED;

  int blk = blockIdx.x;
  if (p.remap) blk = (blk & 7) * (p.nblocks >> 3) + (blk >> 3);
  // (batch row, channel group) and, for a split sequence, the chunk
  int64_t bg = blk, kchunk = 0;
  if (p.nchunks > 1) {
    const int64_t nbg = p.nblocks / p.nchunks;
    kchunk = blk / nbg;
    bg = blk % nbg;
  }
  const int64_t b = bg / p.ngroups;
  const int64_t grp = bg % p.ngroups;
  const int64_t e0 = grp * 16;
  const int64_t tv0 = kchunk * p.chunk_len;                      // the chunk's virtual steps [tv0, tv1)
  const int64_t tv1 = L - tv0 < p.chunk_len ? L : tv0 + p.chunk_len;
  const int64_t R = (tv1 - tv0 + RT - 1) / RT;                   // rounds of the chunk
  const int64_t r0 = tv0 / RT;                                   // its first round in the sweep

  const int64_t e = e0 + ch;
  const bool ch_ok = e < ED;
  const int64_t ec = ch_ok ? e : ED - 1;
  float A2[4], Ar[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    Ar[j] = p.A[ec * 16 + 4 * g + j];
    A2[j] = Ar[j] * kLog2e;
  }
  const float Dv = (p.D && ch_ok) ? p.D[e] : 0.f;

  BwdStager<T, RT, VEC, REV, OPTS> st;
  st.init(tid, b, e0, ED, L, tv0, tv1);
  st.load_bias(p);
  // checkpoint of round rr of the chunk for this lane's 4 states
  auto ck = [&](int64_t rr) { return p.ckpt + ((b * p.rounds + r0 + rr) * p.EDp + e) * 16 + 4 * g; };

  // the states entering the chunk: the forward state before its first step
  // (h0 at the sweep's start) and the adjoint after its last step (dh_last
  // at the sweep's end); a later (earlier) chunk folds the aggregates of the
  // chunks before (after) it onto them
  float hstart[4] = {0.f, 0.f, 0.f, 0.f}, kend[4] = {0.f, 0.f, 0.f, 0.f};
  if (p.h0 && ch_ok) {
    const float4 v = *reinterpret_cast<const float4*>(p.h0 + (b * ED + e) * 16 + 4 * g);
    hstart[0] = v.x, hstart[1] = v.y, hstart[2] = v.z, hstart[3] = v.w;
  }
  if (p.dh_last && ch_ok) {
    const float4 v = *reinterpret_cast<const float4*>(p.dh_last + (b * ED + e) * 16 + 4 * g);
    kend[0] = v.x, kend[1] = v.y, kend[2] = v.z, kend[3] = v.w;
  }
  if (p.nchunks > 1) chunk_entry_states(p, bg, kchunk, ch, g, A2, hstart, kend);
  if (p.ck_given && kchunk > 0) {
    // the forward scan's checkpoint of the chunk's first round (chunks start
    // on round boundaries)
    const float4 v = *reinterpret_cast<const float4*>(ck(0));
    hstart[0] = v.x, hstart[1] = v.y, hstart[2] = v.z, hstart[3] = v.w;
  }

  // ---- sweep 1: forward round aggregates -> checkpoints --------------------
  // (not when the caller passes the forward scan's checkpoints)
  if (R > 1 && !p.ck_given) {
    float hc[4] = {hstart[0], hstart[1], hstart[2], hstart[3]};  // state entering the round (wave SEG-1)
    st.template prefetch<false>(p, 0);
    st.template commit<false>(p, tile[0]);
    __syncthreads();
    for (int64_t r = 0; r + 1 < R; ++r) {
      rotate_priority(r, p.rot_ncu);
      BwdTile<RT>& cur = tile[r & 1];
      BwdTile<RT>& nxt = tile[(r + 1) & 1];
      if (r + 2 < R) st.template prefetch<false>(p, r + 1);
      float hl[4], sd;
#pragma unroll
      for (int i = 0; i < TS; ++i) {
        const int row = wave * TS + i;
        const float dt = cur.dt[row][ch], dxv = dt * cur.xv[row][ch];
        const float bq = cur.bc[row][q].x;
        sd = i == 0 ? dt : sd + dt;
        const float bb[4] = {quad_bcast<0>(bq), quad_bcast<1>(bq), quad_bcast<2>(bq), quad_bcast<3>(bq)};
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const float bv = dxv * bb[j];
          hl[j] = i == 0 ? bv : __builtin_fmaf(__builtin_amdgcn_exp2f(dt * A2[j]), hl[j], bv);
        }
      }
      fa.A[wave][lane] = make_float4(__builtin_amdgcn_exp2f(A2[0] * sd), __builtin_amdgcn_exp2f(A2[1] * sd),
                                     __builtin_amdgcn_exp2f(A2[2] * sd), __builtin_amdgcn_exp2f(A2[3] * sd));
      fa.H[wave][lane] = make_float4(hl[0], hl[1], hl[2], hl[3]);
      __syncthreads();
      if (wave == SEG - 1) {
        for (int k = 0; k < SEG; ++k) {
          const float4 Ak = fa.A[k][lane], Hk = fa.H[k][lane];
          hc[0] = __builtin_fmaf(Ak.x, hc[0], Hk.x);
          hc[1] = __builtin_fmaf(Ak.y, hc[1], Hk.y);
          hc[2] = __builtin_fmaf(Ak.z, hc[2], Hk.z);
          hc[3] = __builtin_fmaf(Ak.w, hc[3], Hk.w);
        }
        *reinterpret_cast<float4*>(ck(r + 1)) = make_float4(hc[0], hc[1], hc[2], hc[3]);
      }
      if (r + 2 < R) st.template commit<false>(p, nxt);
      __syncthreads();
    }
  }

  // ---- sweep 2: rounds in decreasing order --------------------------------
  double dA[4] = {0.0, 0.0, 0.0, 0.0};  // float32 within a round, float64 across rounds
  double dDacc = 0.0;
  float kcar[4] = {0.f, 0.f, 0.f, 0.f};  // adjoint carry out of round 0 (wave 0)
  // the adjoint carry entering the last round: the final state's gradient
  // (padded steps past L have a = 1 and no output, so it reaches step L-1 unchanged)
  if (wave == 0) fa.kc[R & 1][lane] = make_float4(kend[0], kend[1], kend[2], kend[3]);
  st.template prefetch<true>(p, R - 1);
  st.template commit<true>(p, tile[(R - 1) & 1]);
  __syncthreads();
  for (int64_t r = R - 1; r >= 0; --r) {
    rotate_priority(r, p.rot_ncu);
    BwdTile<RT>& cur = tile[r & 1];
    BwdTile<RT>& nxt = tile[(r + 1) & 1];  // round r-1 has the other parity
    if (r >= 1) st.template prefetch<true>(p, r - 1);
    if (r + 1 < R) {
      store_colsums<T, RT, REV>(p, cs, tid, b, grp, tv0, tv1, r + 1);
      st.store_grads(p, nxt, r + 1);  // dx, ddelta of round r+1 (tile of the same parity)
    }

    // forward local pass from a zero state
    float av[TS][4], hv[TS][4];  // a_t; b_t, then h_{t-1}
    float hl[4], sd;
#pragma unroll
    for (int i = 0; i < TS; ++i) {
      const int row = wave * TS + i;
      const float dt = cur.dt[row][ch], dxv = dt * cur.xv[row][ch];
      const float bq = cur.bc[row][q].x;
      sd = i == 0 ? dt : sd + dt;
      const float bb[4] = {quad_bcast<0>(bq), quad_bcast<1>(bq), quad_bcast<2>(bq), quad_bcast<3>(bq)};
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        av[i][j] = __builtin_amdgcn_exp2f(dt * A2[j]);
        hv[i][j] = dxv * bb[j];
        hl[j] = i == 0 ? hv[i][j] : __builtin_fmaf(av[i][j], hl[j], hv[i][j]);
      }
    }
    const float4 Aseg = make_float4(__builtin_amdgcn_exp2f(A2[0] * sd), __builtin_amdgcn_exp2f(A2[1] * sd),
                                    __builtin_amdgcn_exp2f(A2[2] * sd), __builtin_amdgcn_exp2f(A2[3] * sd));
    fa.A[wave][lane] = Aseg;
    fa.H[wave][lane] = make_float4(hl[0], hl[1], hl[2], hl[3]);
    __syncthreads();

    // state entering the segment: the round's checkpoint through segments 0 .. wave-1
    float hin[4] = {hstart[0], hstart[1], hstart[2], hstart[3]};
    if (r > 0) {
      const float4 v = *reinterpret_cast<const float4*>(ck(r));
      hin[0] = v.x, hin[1] = v.y, hin[2] = v.z, hin[3] = v.w;
    }
    for (int k = 0; k < wave; ++k) {
      const float4 Ak = fa.A[k][lane], Hk = fa.H[k][lane];
      hin[0] = __builtin_fmaf(Ak.x, hin[0], Hk.x);
      hin[1] = __builtin_fmaf(Ak.y, hin[1], Hk.y);
      hin[2] = __builtin_fmaf(Ak.z, hin[2], Hk.z);
      hin[3] = __builtin_fmaf(Ak.w, hin[3], Hk.w);
    }
    // forward replay: hv[i] <- h_{t-1} of step i; hin ends as the segment's last state
#pragma unroll
    for (int i = 0; i < TS; ++i) {
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const float hp = hin[j];
        hin[j] = __builtin_fmaf(av[i][j], hin[j], hv[i][j]);
        hv[i][j] = hp;
      }
    }

    // adjoint local pass from a zero carry: k at the segment start
    float kl[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int i = TS - 1; i >= 0; --i) {
      const int row = wave * TS + i;
      const float dyv = cur.dy[row][ch];
      const float cq = cur.bc[row][q].y;
      add_c_dy(kl, cq, dyv);
#pragma unroll
      for (int j = 0; j < 4; ++j) kl[j] *= av[i][j];
    }
    fa.K[wave][lane] = make_float4(kl[0], kl[1], kl[2], kl[3]);
    __syncthreads();

    // adjoint carry entering the segment's end: the next round's carry through
    // segments SEG-1 .. wave+1
    const float4 k0 = fa.kc[(r + 1) & 1][lane];
    float kin[4] = {k0.x, k0.y, k0.z, k0.w};
    for (int k = SEG - 1; k > wave; --k) {
      const float4 Ak = fa.A[k][lane], Kk = fa.K[k][lane];
      kin[0] = __builtin_fmaf(Ak.x, kin[0], Kk.x);
      kin[1] = __builtin_fmaf(Ak.y, kin[1], Kk.y);
      kin[2] = __builtin_fmaf(Ak.z, kin[2], Kk.z);
      kin[3] = __builtin_fmaf(Ak.w, kin[3], Kk.w);
    }

    // adjoint replay and the gradient terms of every step
    const bool writer = g == 0;  // one lane per channel writes dx, ddelta to the tile
    float dAr[4] = {0.f, 0.f, 0.f, 0.f}, dDr = 0.f;
    float hnext[4] = {hin[0], hin[1], hin[2], hin[3]};  // h_t of the step being processed
#pragma unroll
    for (int i = TS - 1; i >= 0; --i) {
      const int row = wave * TS + i;
      const float dt = cur.dt[row][ch], xv = cur.xv[row][ch], dyv = cur.dy[row][ch];
      const float dxv = dt * xv;
      const float2 bcv = cur.bc[row][q];
      add_c_dy(kin, bcv.y, dyv);                  // kin <- g_t
      const float s1 = dot_quad(bcv.x, kin);         // sum_n g B (this lane's 4 states)
      float s2 = 0.f, pv[8];
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        pv[j] = dxv * kin[j];                     // dB term
        pv[4 + j] = dyv * hnext[j];               // dC term
        kin[j] *= av[i][j];                       // k_t = a_t g_t
        const float qv = kin[j] * hv[i][j];       // g a h_{t-1}
        s2 = __builtin_fmaf(Ar[j], qv, s2);
        dAr[j] = __builtin_fmaf(dt, qv, dAr[j]);
        hnext[j] = hv[i][j];
      }
      dDr = __builtin_fmaf(dyv, xv, dDr);
      float s1r = s1;
      bank_sum2(s1r, s2);
      if (writer) {
        // dx and ddelta of the step replace x and dy in the round's tile (this
        // step has read them; no later step reads this row); the staging
        // threads store them one round later, 4 channels per 16-byte store
        cur.xv[row][ch] = __builtin_fmaf(dt, s1r, Dv * dyv);
        cur.dy[row][ch] = __builtin_fmaf(xv, s1r, s2);
      }
      quad_sum8(pv);
      if (c == 0) {
        *reinterpret_cast<float4*>(&cs.v[row][lrow][0][4 * g]) = make_float4(pv[0], pv[1], pv[2], pv[3]);
        *reinterpret_cast<float4*>(&cs.v[row][lrow][1][4 * g]) = make_float4(pv[4], pv[5], pv[6], pv[7]);
      }
    }
#pragma unroll
    for (int j = 0; j < 4; ++j) dA[j] += static_cast<double>(dAr[j]);
    dDacc += static_cast<double>(dDr);
    if (wave == 0) {
      fa.kc[r & 1][lane] = make_float4(kin[0], kin[1], kin[2], kin[3]);
#pragma unroll
      for (int j = 0; j < 4; ++j) kcar[j] = kin[j];
    }
    if (r >= 1) st.template commit<true>(p, nxt);
    __syncthreads();
  }
  store_colsums<T, RT, REV>(p, cs, tid, b, grp, tv0, tv1, 0);
  st.store_grads(p, tile[0], 0);

  // ---- per-workgroup results ----------------------------------------------
  // (a later chunk's entering-state gradient stays inside the sweep)
  if (p.dh0 && kchunk == 0 && wave == 0 && ch_ok)
    *reinterpret_cast<float4*>(p.dh0 + (b * ED + e) * 16 + 4 * g) = make_float4(kcar[0], kcar[1], kcar[2], kcar[3]);
  const int64_t prow = b * p.nchunks + kchunk;  // partial row of dA, dD, ddt_bias
  // dA and dD: sums over the waves' segments, then one partial per batch row
  double* red = reinterpret_cast<double*>(&fa);  // [SEG][5][64]; the fold area is free now
  static_assert(sizeof(BwdFold<SEG>) >= sizeof(double) * SEG * 5 * 64, "reduction area");
#pragma unroll
  for (int j = 0; j < 4; ++j) red[(wave * 5 + j) * 64 + lane] = dA[j];
  red[(wave * 5 + 4) * 64 + lane] = dDacc;
  __syncthreads();
  if (wave == 0) {
#pragma unroll
    for (int j = 0; j < 5; ++j) {
      double s = red[j * 64 + lane];
      for (int k = 1; k < SEG; ++k) s += red[(k * 5 + j) * 64 + lane];
      if (j < 4) p.pA[(prow * p.EDp + e) * 16 + 4 * g + j] = s;
      else if (g == 0) p.pD[prow * p.EDp + e] = s;
    }
  }
  // ddt_bias: the step-size tasks' sums, added over the round's rows in row
  // order (the column-sum tile is free since the barrier above)
  if (OPTS && p.pDB) {
    double* dbs = reinterpret_cast<double*>(&cs);  // [RT rows][16 channels]
    static_assert(sizeof(ColSums<RT>) >= sizeof(double) * RT * 16, "reduction area");
    if (st.is_xd) {
      dbs[st.row * 16 + 4 * st.chk + 0] = st.dbacc[0];
      dbs[st.row * 16 + 4 * st.chk + 1] = st.dbacc[1];
      dbs[st.row * 16 + 4 * st.chk + 2] = st.dbacc[2];
      dbs[st.row * 16 + 4 * st.chk + 3] = st.dbacc[3];
    }
    __syncthreads();
    if (tid < 16) {
      double s = 0.0;
      for (int r = 0; r < RT; ++r) s += dbs[r * 16 + tid];
      p.pDB[prow * p.EDp + e0 + tid] = s;
    }
  }
}

// dB, dC: sum of the channel groups' partials. A workgroup covers 64 float4
// positions; its 4 waves each add up one quarter of the groups in group
// order, and the quarters are added in order (a fixed order: deterministic).
template <typename T>
__global__ __launch_bounds__(256) void bwd_reduce_bc_kernel(const float* __restrict__ pB,
                                                            const float* __restrict__ pC, T* dB, T* dC, int64_t n4,
                                                            int ngroups) {
  __shared__ float4 part[4][64];
  const int lane = threadIdx.x & 63, quarter = threadIdx.x >> 6;
  const int64_t i = blockIdx.x * static_cast<int64_t>(64) + lane;  // float4 index over dB then dC
  const bool ok = i < 2 * n4;
  const bool isC = i >= n4;
  const int64_t k = isC ? i - n4 : i;
  const float4* src = reinterpret_cast<const float4*>(isC ? pC : pB) + k;
  const int per = (ngroups + 3) / 4;
  const int g0 = quarter * per, g1 = min(ngroups, g0 + per);
  float4 s = make_float4(0.f, 0.f, 0.f, 0.f);
  // the groups in order either way; more loads in flight pay off only for
  // long quarters
  if (ok && g1 - g0 >= 32) {
#pragma unroll 16
    for (int gi = g0; gi < g1; ++gi) {
      const float4 v = src[gi * n4];
      s = make_float4(s.x + v.x, s.y + v.y, s.z + v.z, s.w + v.w);
    }
  } else if (ok) {
#pragma unroll 8
    for (int gi = g0; gi < g1; ++gi) {
      const float4 v = src[gi * n4];
      s = make_float4(s.x + v.x, s.y + v.y, s.z + v.z, s.w + v.w);
    }
  }
  part[quarter][lane] = s;
  __syncthreads();
  if (quarter == 0 && ok) {
#pragma unroll
    for (int h = 1; h < 4; ++h) {
      const float4 v = part[h][lane];
      s = make_float4(s.x + v.x, s.y + v.y, s.z + v.z, s.w + v.w);
    }
    Vec4<T>::store((isC ? dC : dB) + 4 * k, s);
  }
}

// dA, dD: sum of the batch rows' partials, in row order (the bidirectional
// backward has 2 Bs rows of dA partials: the forward-time scan's, then the
// reverse-time scan's; dD comes from the forward-time scan alone).
__global__ void bwd_reduce_ad_kernel(const double* __restrict__ pA, const double* __restrict__ pD,
                                     const double* __restrict__ pDB, float* dA, float* dD, float* ddt_bias,
                                     int64_t rowsA, int64_t rowsD, int64_t ED, int64_t EDp) {
  const int64_t i = blockIdx.x * static_cast<int64_t>(blockDim.x) + threadIdx.x;
  if (i < ED * 16) {
    const int64_t e = i >> 4, n = i & 15;
    double s = 0.0;
    for (int64_t b = 0; b < rowsA; ++b) s += pA[(b * EDp + e) * 16 + n];
    dA[i] = static_cast<float>(s);
  } else if (dD && i < ED * 17) {
    const int64_t e = i - ED * 16;
    double s = 0.0;
    for (int64_t b = 0; b < rowsD; ++b) s += pD[b * EDp + e];
    dD[e] = static_cast<float>(s);
  } else if (ddt_bias && i >= ED * 17 && i < ED * 18) {
    // ddt_bias: the sum of the rows' partials (both directions for the bidirectional scan)
    const int64_t e = i - ED * 17;
    double s = 0.0;
    for (int64_t b = 0; b < rowsA; ++b) s += pDB[b * EDp + e];
    ddt_bias[e] = static_cast<float>(s);
  }
}

// The output gate: y = y' silu(z), y' the ungated output (held in dz on
// entry, recomputed by the forward scan). dz = dy y' silu'(z) with
// silu'(z) = s (1 + z (1 - s)), s = sigmoid(z), written over y'; the scan's
// own output gradient is dy silu(z) (dyg, kept in float32: it is summed
// over many steps and channels, where a rounding to bf16 would add up).
template <typename T>
__global__ void gate_bwd_kernel(const T* __restrict__ dy, const T* __restrict__ z, T* dz, float* __restrict__ dyg,
                                int64_t n) {
  for (int64_t i = blockIdx.x * static_cast<int64_t>(blockDim.x) + threadIdx.x; i < n;
       i += static_cast<int64_t>(gridDim.x) * blockDim.x) {
    const float zv = to_f32(z[i]), g = to_f32(dy[i]), yp = to_f32(dz[i]);
    const float sg = 1.f / (1.f + __expf(-zv));
    dz[i] = from_f32<T>(g * yp * sg * (1.f + zv * (1.f - sg)));
    dyg[i] = g * zv * sg;
  }
}

// ---------------------------------------------------------------------------
// host side
// ---------------------------------------------------------------------------
struct BwdLayout {
  int64_t rounds, ngroups, EDp;
  int64_t nchunks, chunk_len;  // split sweep: chunks per (batch row, channel group) and their length
  size_t ckpt_off, pB_off, pC_off, pA_off, pD_off, pDB_off, part_off, agg_off, bytes;
};

size_t align256(size_t v) { return (v + 255) & ~static_cast<size_t>(255); }

// Workspace: round checkpoints, the dB / dC partials of every channel group,
// the dA / dD partials of every batch row; the bidirectional backward keeps
// both directions' partials (dirs = 2) and, for bf16 outputs, the forward-time
// scan's dx and ddelta as float32 (part_f32).
bool bwd_layout(int64_t Bs, int64_t L, int64_t ED, BwdLayout* lo, bool bidir = false, bool part_f32 = false) {
  const int64_t dirs = bidir ? 2 : 1;
  lo->rounds = (L + kBRT - 1) / kBRT;
  lo->ngroups = (ED + 15) / 16;
  lo->EDp = lo->ngroups * 16;
  // A long sweep with fewer than two (batch row, channel group) pairs per
  // compute unit is cut into chunks (each at least 16 rounds, about three
  // workgroups per CU in all), as the forward scan does.
  lo->nchunks = 1;
  lo->chunk_len = L;
  const int64_t nbg = Bs * lo->ngroups, ncu = device_cus();
  if (ncu > 0 && nbg > 0 && nbg < 2 * ncu) {
    const int64_t k = std::min<int64_t>(3 * ncu / nbg, L / (16 * kBRT));
    if (k >= 2) {
      lo->chunk_len = ((L + k - 1) / k + kBRT - 1) / kBRT * kBRT;
      lo->nchunks = (L + lo->chunk_len - 1) / lo->chunk_len;
    }
  }
  const int64_t rows = Bs * lo->nchunks;  // dA / dD / ddt_bias partial rows per direction
  // every count below is checked against overflow of size_t arithmetic
  const double total = 4.0 * (static_cast<double>(Bs) * lo->rounds * lo->EDp * 16 +
                              2.0 * dirs * lo->ngroups * Bs * L * 16 + 2.0 * dirs * rows * lo->EDp * 18 +
                              (part_f32 ? 2.0 * Bs * L * ED : 0.0) +
                              (lo->nchunks > 1 ? dirs * 544.0 * nbg * lo->nchunks : 0.0)) +
                       7 * 256.0;
  if (total > 9.0e18) return false;
  size_t off = 0;
  lo->ckpt_off = off;
  off = align256(off + static_cast<size_t>(Bs * lo->rounds * lo->EDp * 16) * 4);
  lo->pB_off = off;
  off = align256(off + static_cast<size_t>(dirs * lo->ngroups * Bs * L * 16) * 4);
  lo->pC_off = off;
  off = align256(off + static_cast<size_t>(dirs * lo->ngroups * Bs * L * 16) * 4);
  lo->pA_off = off;
  off = align256(off + static_cast<size_t>(dirs * rows * lo->EDp * 16) * 8);
  lo->pD_off = off;
  off = align256(off + static_cast<size_t>(dirs * rows * lo->EDp) * 8);
  lo->pDB_off = off;
  off = align256(off + static_cast<size_t>(dirs * rows * lo->EDp) * 8);
  lo->part_off = off;
  if (part_f32) off = align256(off + static_cast<size_t>(2 * Bs * L * ED) * 4);
  // chunk aggregates per direction: [slot][16] float64 sums of delta', then
  // [slot][16][16] forward end states and [slot][16][16] adjoint start states
  lo->agg_off = off;
  if (lo->nchunks > 1) off = align256(off + static_cast<size_t>(dirs * nbg * lo->nchunks) * (16 * 8 + 2 * 256 * 4));
  lo->bytes = off;
  return true;
}

struct BwdSizes {
  int64_t seq, bc, state, elem;
};

// Bs, L and ED may be zero (empty tensors); N must be 16.
int bwd_check_sizes(int64_t Bs, int64_t L, int64_t ED, int64_t N, int dtype, BwdSizes* s) {
  if (Bs < 0 || L < 0 || ED < 0 || N <= 0) return SSM_ERR_DIM;
  int64_t t;
  if (!mul_nn(Bs, L, &t) || !mul_nn(t, ED, &s->seq) || !mul_nn(t, N, &s->bc)) return SSM_ERR_DIM;
  if (!mul_nn(Bs, ED, &t) || !mul_nn(t, N, &s->state)) return SSM_ERR_DIM;
  if (s->seq > INT64_MAX / 8 || s->state > INT64_MAX / 8 || s->bc > INT64_MAX / 8 / ((ED + 15) / 16 + 1))
    return SSM_ERR_DIM;
  if (dtype != SSM_F32 && dtype != SSM_BF16) return SSM_ERR_UNSUPPORTED;
  if (N != 16) return SSM_ERR_UNSUPPORTED;
  s->elem = dtype == SSM_F32 ? 4 : 2;
  return SSM_OK;
}

// With the gate the workspace also holds dy silu(z) (float32, one value per
// element of x) after the backward's own area; the forward scan that
// recomputes the ungated output runs first and borrows the start of it.
// *gate_off: where dy silu(z) starts.
size_t gated_bytes(int64_t Bs, int64_t L, int64_t ED, int64_t N, int dtype, bool bidir, const BwdSizes& s,
                   size_t bwd_bytes, size_t* gate_off) {
  const size_t fwd = ssm_scan_workspace_bytes(Bs, L, ED, N, dtype, bidir ? 1 : 0);
  *gate_off = align256(std::max(bwd_bytes, fwd));
  return *gate_off + align256(static_cast<size_t>(s.seq * 4));
}

size_t bwd_workspace_bytes(int64_t Bs, int64_t L, int64_t ED, int64_t N, int dtype, bool bidir, bool gate) {
  BwdSizes s;
  BwdLayout lo;
  if (bwd_check_sizes(Bs, L, ED, N, dtype, &s) != SSM_OK || s.seq == 0 ||
      !bwd_layout(Bs, L, ED, &lo, bidir, bidir && dtype == SSM_BF16))
    return 0;
  size_t off;
  return gate ? gated_bytes(Bs, L, ED, N, dtype, bidir, s, lo.bytes, &off) : lo.bytes;
}

// The carried states of a call and their gradients: the reverse direction's
// initial state g0 (bidirectional), the final states' gradients dh_last and
// dg_first (bidirectional) given by the caller, and dg0 (bidirectional) out.
struct StateArgs {
  const float* g0;
  const float* dh_last;
  const float* dg_first;
  float* dg0;
  const float* ckpt;  // the forward scan's round checkpoints, or nullptr
  size_t ck_bytes;
};

int bwd_validate(const void* x, const void* delta, const float* A, const void* B, const void* C, const float* D,
                 const float* h0, const ssm_scan_options* opts, const void* dy, const void* dx, const void* ddelta,
                 const float* dA, const void* dB, const void* dC, const float* dD, const float* dh0,
                 const float* ddt_bias, const void* dz, const StateArgs& sa, int64_t Bs, int64_t L, int64_t ED,
                 int64_t N, int dtype, const void* ws, size_t ws_bytes, bool bidir, BwdSizes* s, size_t* gate_off) {
  int rc = bwd_check_sizes(Bs, L, ED, N, dtype, s);
  if (rc != SSM_OK) return rc;
  if (opts && !(opts->dt_min <= opts->dt_max)) return SSM_ERR_ARG;  // also catches NaN
  const float* dt_bias = opts ? opts->dt_bias : nullptr;
  const void* z = opts ? opts->z : nullptr;
  if (!z) dz = nullptr;  // dz is written only with the gate
  // a buffer with no elements may be NULL
  if ((s->seq > 0 && (!x || !delta || !dy || !dx || !ddelta || (z && !dz))) ||
      (s->bc > 0 && (!B || !C || !dB || !dC)) || (ED > 0 && (!A || !dA)))
    return SSM_ERR_NULL;
  const void* ptrs[] = {x,  delta, A,      B,        C,  D,  h0,       dt_bias,        z,     dy,    dx,
                        ddelta, dA, dB, dC, dD, dh0, ddt_bias, dz, ws, sa.g0, sa.dh_last, sa.dg_first, sa.dg0};
  for (const void* q : ptrs)
    if (q && !aligned16(q)) return SSM_ERR_UNSUPPORTED;
  BwdLayout lo;
  if (!bwd_layout(Bs, L, ED, &lo, bidir, bidir && dtype == SSM_BF16)) return SSM_ERR_DIM;
  // the forward scan's checkpoints: (Bs, rounds, 16 ceil(ED / 16), 16) float32
  const int64_t ck_need = sa.ckpt && s->seq > 0 ? Bs * lo.rounds * lo.EDp * 16 * 4 : 0;
  if (sa.ckpt && !aligned16(sa.ckpt)) return SSM_ERR_UNSUPPORTED;
  if (ck_need > 0 && sa.ck_bytes < static_cast<size_t>(ck_need)) return SSM_ERR_WORKSPACE;
  if (s->seq == 0) lo.bytes = 0;  // nothing is scanned: no workspace
  else if (z) lo.bytes = gated_bytes(Bs, L, ED, N, dtype, bidir, *s, lo.bytes, gate_off);
  if (lo.bytes > 0 && (!ws || ws_bytes < lo.bytes)) return SSM_ERR_WORKSPACE;
  const Range in[] = {rng(x, s->seq * s->elem), rng(delta, s->seq * s->elem), rng(A, ED * N * 4),
                      rng(B, s->bc * s->elem),  rng(C, s->bc * s->elem),      rng(D, D ? ED * 4 : 0),
                      rng(h0, h0 ? s->state * 4 : 0), rng(dy, s->seq * s->elem), rng(dt_bias, dt_bias ? ED * 4 : 0),
                      rng(z, z ? s->seq * s->elem : 0), rng(sa.g0, sa.g0 ? s->state * 4 : 0),
                      rng(sa.dh_last, sa.dh_last ? s->state * 4 : 0), rng(sa.dg_first, sa.dg_first ? s->state * 4 : 0),
                      rng(sa.ckpt, ck_need)};
  const Range out[] = {rng(dx, s->seq * s->elem), rng(ddelta, s->seq * s->elem), rng(dA, ED * N * 4),
                       rng(dB, s->bc * s->elem),  rng(dC, s->bc * s->elem),      rng(dD, dD ? ED * 4 : 0),
                       rng(dh0, dh0 ? s->state * 4 : 0), rng(ddt_bias, ddt_bias ? ED * 4 : 0),
                       rng(dz, dz ? s->seq * s->elem : 0), rng(ws, static_cast<int64_t>(lo.bytes)),
                       rng(sa.dg0, sa.dg0 ? s->state * 4 : 0)};
  constexpr int nout = sizeof(out) / sizeof(out[0]);
  for (int i = 0; i < nout; ++i) {
    if (out[i].hi == out[i].lo) continue;
    for (const Range& r : in)
      if (r.hi > r.lo && overlap(out[i], r)) return SSM_ERR_ALIAS;
    for (int j = i + 1; j < nout; ++j)
      if (out[j].hi > out[j].lo && overlap(out[i], out[j])) return SSM_ERR_ALIAS;
  }
  return SSM_OK;
}

template <typename T, bool REV, bool FWD>
void launch_agg(const BwdArgs<T>& a, int64_t nblk, bool vec, hipStream_t stream) {
  if (a.dt_pre) {
    if (vec)
      hipLaunchKernelGGL((bwd_chunk_agg_kernel<T, kBSEG, kBTS, true, REV, true, FWD>), dim3(nblk), dim3(64 * kBSEG), 0,
                         stream, a);
    else
      hipLaunchKernelGGL((bwd_chunk_agg_kernel<T, kBSEG, kBTS, false, REV, true, FWD>), dim3(nblk), dim3(64 * kBSEG),
                         0, stream, a);
  } else {
    if (vec)
      hipLaunchKernelGGL((bwd_chunk_agg_kernel<T, kBSEG, kBTS, true, REV, false, FWD>), dim3(nblk), dim3(64 * kBSEG),
                         0, stream, a);
    else
      hipLaunchKernelGGL((bwd_chunk_agg_kernel<T, kBSEG, kBTS, false, REV, false, FWD>), dim3(nblk), dim3(64 * kBSEG),
                         0, stream, a);
  }
}

template <typename T, bool REV>
void launch_bwd_kernel(const BwdArgs<T>& a, int64_t nblk, size_t dyn, bool vec, hipStream_t stream) {
  if (a.nchunks > 1) {
    // the chunks' aggregates first (same grid; the launch order on the stream
    // joins them); with the forward scan's checkpoints, the adjoint's only
    if (a.ck_given)
      launch_agg<T, REV, false>(a, nblk, vec, stream);
    else
      launch_agg<T, REV, true>(a, nblk, vec, stream);
  }
  if (a.dt_pre) {
    if (vec)
      hipLaunchKernelGGL((scan_bwd_kernel<T, kBSEG, kBTS, true, REV, true>), dim3(nblk), dim3(64 * kBSEG), dyn, stream, a);
    else
      hipLaunchKernelGGL((scan_bwd_kernel<T, kBSEG, kBTS, false, REV, true>), dim3(nblk), dim3(64 * kBSEG), dyn, stream, a);
  } else {
    if (vec)
      hipLaunchKernelGGL((scan_bwd_kernel<T, kBSEG, kBTS, true, REV, false>), dim3(nblk), dim3(64 * kBSEG), dyn, stream, a);
    else
      hipLaunchKernelGGL((scan_bwd_kernel<T, kBSEG, kBTS, false, REV, false>), dim3(nblk), dim3(64 * kBSEG), dyn, stream, a);
  }
}

template <typename T>
int launch_bwd(const void* x, const void* delta, const float* A, const void* B, const void* C, const float* D,
               const float* h0, const ssm_scan_options* opts, const void* dy, void* dx, void* ddelta, float* dA,
               void* dB, void* dC, float* dD, float* dh0, float* ddt_bias, const StateArgs& sa, int64_t Bs,
               int64_t L, int64_t ED, void* ws, bool bidir, const float* dyf, hipStream_t stream) {
  const bool part_f32 = bidir && !std::is_same<T, float>::value;
  BwdLayout lo;
  bwd_layout(Bs, L, ED, &lo, bidir, part_f32);
  const int64_t nbg = Bs * lo.ngroups;
  const int64_t nblk = nbg * lo.nchunks;
  if (nblk > INT32_MAX / 2) return SSM_ERR_DIM;
  const int64_t rows = Bs * lo.nchunks;  // dA / dD / ddt_bias partial rows per direction
  char* w = static_cast<char*>(ws);
  BwdArgs<T> a;
  a.x = static_cast<const T*>(x);
  a.dl = static_cast<const T*>(delta);
  a.A = A;
  a.B = static_cast<const T*>(B);
  a.C = static_cast<const T*>(C);
  a.D = D;
  a.h0 = h0;
  a.dh_last = sa.dh_last;
  a.dt_bias = opts ? opts->dt_bias : nullptr;
  a.dt_softplus = opts && opts->dt_softplus ? 1 : 0;
  a.dt_min = opts ? opts->dt_min : -INFINITY;
  a.dt_max = opts ? opts->dt_max : INFINITY;
  // (a requested ddt_bias takes the options path: with no option the map is
  // the identity and ddt_bias is the sum of ddelta)
  // the gated output gradient (dyf) is read by the options kernels too
  a.dt_pre = (a.dt_bias || a.dt_softplus || a.dt_min > -INFINITY || a.dt_max < INFINITY || ddt_bias || dyf) ? 1 : 0;
  a.dyf = dyf;
  a.pDB = ddt_bias ? reinterpret_cast<double*>(w + lo.pDB_off) : nullptr;
  a.dy = static_cast<const T*>(dy);
  a.dx = static_cast<T*>(dx);
  a.ddl = static_cast<T*>(ddelta);
  a.dh0 = dh0;
  // the kernels only read checkpoints that the caller passes
  a.ckpt = sa.ckpt ? const_cast<float*>(sa.ckpt) : reinterpret_cast<float*>(w + lo.ckpt_off);
  a.ck_given = sa.ckpt ? 1 : 0;
  a.pB = reinterpret_cast<float*>(w + lo.pB_off);
  a.pC = reinterpret_cast<float*>(w + lo.pC_off);
  a.pA = reinterpret_cast<double*>(w + lo.pA_off);
  a.pD = reinterpret_cast<double*>(w + lo.pD_off);
  a.Bs = Bs;
  a.L = L;
  a.ED = ED;
  a.EDp = lo.EDp;
  a.rounds = lo.rounds;
  a.ngroups = static_cast<int>(lo.ngroups);
  a.nblocks = static_cast<int>(nblk);
  a.remap = (nblk % 8 == 0) ? 1 : 0;
  a.rot_ncu = rotation_cus(nblk);
  float* part = reinterpret_cast<float*>(w + lo.part_off);
  a.part_dx = part_f32 ? part : nullptr;
  a.part_dd = part_f32 ? part + Bs * L * ED : nullptr;
  a.acc_dx = nullptr;
  a.acc_dd = nullptr;
  a.nchunks = static_cast<int>(lo.nchunks);
  a.chunk_len = lo.chunk_len;
  const size_t nslot = static_cast<size_t>(nbg * lo.nchunks);
  char* agg = w + lo.agg_off;
  a.agg_sd = lo.nchunks > 1 ? reinterpret_cast<double*>(agg) : nullptr;
  a.agg_h = lo.nchunks > 1 ? reinterpret_cast<float*>(agg + nslot * 16 * 8) : nullptr;
  a.agg_k = lo.nchunks > 1 ? a.agg_h + nslot * 256 : nullptr;

  const size_t lds = sizeof(BwdTile<kBRT>) * 2 + sizeof(ColSums<kBRT>) + sizeof(BwdFold<kBSEG>) + 16;
  const size_t dyn = spread_lds(nblk, lds, 16 / kBSEG);
  const bool vec = ED % 4 == 0;
  launch_bwd_kernel<T, false>(a, nblk, dyn, vec, stream);
  if (hipGetLastError() != hipSuccess) return SSM_ERR_LAUNCH;
  if (bidir) {
    // the reverse-time scan: from g0 (or zero) at t = L-1, no D, the adjoint
    // entering from dg_first, its own halves of the partials, dx and ddelta
    // added to the forward-time scan's (in order on the stream) and rounded
    // once; its initial state's gradient is dg0
    BwdArgs<T> r = a;
    // the caller's checkpoints are the forward direction's; this scan keeps
    // its own first sweep and workspace checkpoints
    r.ckpt = reinterpret_cast<float*>(w + lo.ckpt_off);
    r.ck_given = 0;
    r.D = nullptr;
    r.h0 = sa.g0;
    r.dh0 = sa.dg0;
    r.dh_last = sa.dg_first;
    r.pB = a.pB + lo.ngroups * Bs * L * 16;
    r.pC = a.pC + lo.ngroups * Bs * L * 16;
    r.pA = a.pA + rows * lo.EDp * 16;
    r.pD = a.pD + rows * lo.EDp;
    r.pDB = a.pDB ? a.pDB + rows * lo.EDp : nullptr;
    if (lo.nchunks > 1) {
      // the reverse-time scan's own chunk aggregates
      char* agg_r = agg + nslot * (16 * 8 + 2 * 256 * 4);
      r.agg_sd = reinterpret_cast<double*>(agg_r);
      r.agg_h = reinterpret_cast<float*>(agg_r + nslot * 16 * 8);
      r.agg_k = r.agg_h + nslot * 256;
    }
    r.part_dx = nullptr;
    r.part_dd = nullptr;
    r.acc_dx = part_f32 ? a.part_dx : static_cast<const float*>(dx);
    r.acc_dd = part_f32 ? a.part_dd : static_cast<const float*>(ddelta);
    launch_bwd_kernel<T, true>(r, nblk, dyn, vec, stream);
    if (hipGetLastError() != hipSuccess) return SSM_ERR_LAUNCH;
  }

  const int64_t n4 = Bs * L * 4;  // float4s per dB (or dC)
  if ((2 * n4 + 63) / 64 > INT32_MAX) return SSM_ERR_DIM;
  hipLaunchKernelGGL(bwd_reduce_bc_kernel<T>, dim3(static_cast<unsigned>((2 * n4 + 63) / 64)), dim3(256), 0,
                     stream, a.pB, a.pC, static_cast<T*>(dB), static_cast<T*>(dC), n4,
                     static_cast<int>(bidir ? 2 * lo.ngroups : lo.ngroups));
  if (hipGetLastError() != hipSuccess) return SSM_ERR_LAUNCH;
  hipLaunchKernelGGL(bwd_reduce_ad_kernel, dim3(static_cast<unsigned>((ED * 18 + 255) / 256)), dim3(256), 0, stream,
                     a.pA, a.pD, a.pDB, dA, dD, ddt_bias, bidir ? 2 * rows : rows, rows, ED, lo.EDp);
  return hipGetLastError() == hipSuccess ? SSM_OK : SSM_ERR_LAUNCH;
}

int run_bwd(const void* x, const void* delta, const float* A, const void* B, const void* C, const float* D,
            const float* h0, const ssm_scan_options* opts, const void* dy, void* dx, void* ddelta, float* dA,
            void* dB, void* dC, float* dD, float* dh0, float* ddt_bias, void* dz, StateArgs sa, int64_t Bs,
            int64_t L, int64_t ED, int64_t N, int dtype, void* workspace, size_t workspace_bytes, void* stream,
            bool bidir) {
  BwdSizes s;
  size_t gate_off = 0;
  if (!bidir) sa.g0 = sa.dg_first = sa.dg0 = nullptr;
  const int rc = bwd_validate(x, delta, A, B, C, D, h0, opts, dy, dx, ddelta, dA, dB, dC, dD, dh0, ddt_bias, dz, sa,
                              Bs, L, ED, N, dtype, workspace, workspace_bytes, bidir, &s, &gate_off);
  if (rc != SSM_OK) return rc;
  hipStream_t st = static_cast<hipStream_t>(stream);
  ssm_scan_options ungated{};
  const float* dyf = nullptr;
  if (opts && opts->z && s.seq > 0) {
    // the gate: recompute the ungated output y' into dz, form dz and
    // dy silu(z), then the backward of y' with that output gradient
    ungated = *opts;
    ungated.z = nullptr;
    const int frc = bidir ? ssm_scan_bidir_fwd(x, delta, A, B, C, D, h0, sa.g0, &ungated, dz, nullptr, nullptr, Bs,
                                               L, ED, N, dtype, workspace, gate_off, stream)
                          : ssm_scan_fwd(x, delta, A, B, C, D, h0, &ungated, dz, nullptr, Bs, L, ED, N, dtype,
                                         workspace, gate_off, stream);
    if (frc != SSM_OK) return frc;
    float* dyg = reinterpret_cast<float*>(static_cast<char*>(workspace) + gate_off);
    const unsigned grid = static_cast<unsigned>(std::min<int64_t>((s.seq + 255) / 256, 8192));
    if (dtype == SSM_F32)
      hipLaunchKernelGGL(gate_bwd_kernel<float>, dim3(grid), dim3(256), 0, st, static_cast<const float*>(dy),
                         static_cast<const float*>(opts->z), static_cast<float*>(dz), dyg, s.seq);
    else
      hipLaunchKernelGGL(gate_bwd_kernel<uint16_t>, dim3(grid), dim3(256), 0, st, static_cast<const uint16_t*>(dy),
                         static_cast<const uint16_t*>(opts->z), static_cast<uint16_t*>(dz), dyg, s.seq);
    if (hipGetLastError() != hipSuccess) return SSM_ERR_LAUNCH;
    dyf = dyg;
    opts = &ungated;
  }
  if (s.seq == 0) {
    // an empty output: every gradient is zero (dB and dC too when there are
    // time steps but no channels), except that over zero steps each final
    // state is its initial state, so dh0 = dh_last and dg0 = dg_first
    const bool ok = fill_async(dA, nullptr, ED * N * 4, st) && fill_async(dD, nullptr, ED * 4, st) &&
                    fill_async(dh0, sa.dh_last, s.state * 4, st) && fill_async(sa.dg0, sa.dg_first, s.state * 4, st) &&
                    fill_async(dB, nullptr, s.bc * s.elem, st) &&
                    fill_async(dC, nullptr, s.bc * s.elem, st) && fill_async(ddt_bias, nullptr, ED * 4, st);
    return ok ? SSM_OK : SSM_ERR_LAUNCH;
  }
  if (dtype == SSM_F32)
    return launch_bwd<float>(x, delta, A, B, C, D, h0, opts, dy, dx, ddelta, dA, dB, dC, dD, dh0, ddt_bias, sa, Bs,
                             L, ED, workspace, bidir, dyf, st);
  return launch_bwd<uint16_t>(x, delta, A, B, C, D, h0, opts, dy, dx, ddelta, dA, dB, dC, dD, dh0, ddt_bias, sa, Bs,
                              L, ED, workspace, bidir, dyf, st);
}

}  // namespace

extern "C" {

size_t ssm_scan_bwd_workspace_bytes(int64_t Bs, int64_t L, int64_t ED, int64_t N, int dtype, int gate) {
  return bwd_workspace_bytes(Bs, L, ED, N, dtype, false, gate != 0);
}

size_t ssm_scan_bidir_bwd_workspace_bytes(int64_t Bs, int64_t L, int64_t ED, int64_t N, int dtype, int gate) {
  return bwd_workspace_bytes(Bs, L, ED, N, dtype, true, gate != 0);
}

int ssm_scan_bwd(const void* x, const void* delta, const float* A, const void* B, const void* C, const float* D,
                 const float* h0, const ssm_scan_options* opts, const void* dy, const float* dh_last, void* dx,
                 void* ddelta, float* dA, void* dB, void* dC, float* dD, float* dh0, float* ddt_bias, void* dz,
                 int64_t Bs, int64_t L, int64_t ED, int64_t N, int dtype, void* workspace, size_t workspace_bytes,
                 void* stream) {
  const StateArgs sa{nullptr, dh_last, nullptr, nullptr, nullptr, 0};
  return run_bwd(x, delta, A, B, C, D, h0, opts, dy, dx, ddelta, dA, dB, dC, dD, dh0, ddt_bias, dz, sa, Bs, L, ED,
                 N, dtype, workspace, workspace_bytes, stream, false);
}

int ssm_scan_bwd_ckpt(const void* x, const void* delta, const float* A, const void* B, const void* C,
                      const float* D, const float* h0, const ssm_scan_options* opts, const void* dy,
                      const float* dh_last, const float* ckpt, size_t ckpt_bytes, void* dx, void* ddelta, float* dA,
                      void* dB, void* dC, float* dD, float* dh0, float* ddt_bias, void* dz, int64_t Bs, int64_t L,
                      int64_t ED, int64_t N, int dtype, void* workspace, size_t workspace_bytes, void* stream) {
  // a NULL ckpt is an error here (ssm_scan_bwd is the call without one),
  // unless there is nothing to scan
  if (!ckpt && Bs > 0 && L > 0 && ED > 0) return SSM_ERR_NULL;
  const StateArgs sa{nullptr, dh_last, nullptr, nullptr, ckpt, ckpt_bytes};
  return run_bwd(x, delta, A, B, C, D, h0, opts, dy, dx, ddelta, dA, dB, dC, dD, dh0, ddt_bias, dz, sa, Bs, L, ED,
                 N, dtype, workspace, workspace_bytes, stream, false);
}

int ssm_scan_bidir_bwd(const void* x, const void* delta, const float* A, const void* B, const void* C,
                       const float* D, const float* h0, const float* g0, const ssm_scan_options* opts, const void* dy,
                       const float* dh_last, const float* dg_first, void* dx, void* ddelta, float* dA, void* dB,
                       void* dC, float* dD, float* dh0, float* dg0, float* ddt_bias, void* dz, int64_t Bs, int64_t L,
                       int64_t ED, int64_t N, int dtype, void* workspace, size_t workspace_bytes, void* stream) {
  const StateArgs sa{g0, dh_last, dg_first, dg0, nullptr, 0};
  return run_bwd(x, delta, A, B, C, D, h0, opts, dy, dx, ddelta, dA, dB, dC, dD, dh0, ddt_bias, dz, sa, Bs, L, ED,
                 N, dtype, workspace, workspace_bytes, stream, true);
}

int ssm_scan_bidir_bwd_ckpt(const void* x, const void* delta, const float* A, const void* B, const void* C,
                            const float* D, const float* h0, const float* g0, const ssm_scan_options* opts,
                            const void* dy, const float* dh_last, const float* dg_first, const float* ckpt,
                            size_t ckpt_bytes, void* dx, void* ddelta, float* dA, void* dB, void* dC, float* dD,
                            float* dh0, float* dg0, float* ddt_bias, void* dz, int64_t Bs, int64_t L, int64_t ED,
                            int64_t N, int dtype, void* workspace, size_t workspace_bytes, void* stream) {
  if (!ckpt && Bs > 0 && L > 0 && ED > 0) return SSM_ERR_NULL;
  const StateArgs sa{g0, dh_last, dg_first, dg0, ckpt, ckpt_bytes};
  return run_bwd(x, delta, A, B, C, D, h0, opts, dy, dx, ddelta, dA, dB, dC, dD, dh0, ddt_bias, dz, sa, Bs, L, ED,
                 N, dtype, workspace, workspace_bytes, stream, true);
}

}  // extern "C"
