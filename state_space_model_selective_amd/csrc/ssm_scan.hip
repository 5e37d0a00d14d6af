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
// 4-wide element access (16-byte float32 / 8-byte bfloat16 vectors)
// ---------------------------------------------------------------------------
template <typename T>
struct Vec4;
template <>
struct Vec4<float> {
  static __device__ __forceinline__ float4 load(const float* p) { return *reinterpret_cast<const float4*>(p); }
  static __device__ __forceinline__ void store(float* p, float4 v) { *reinterpret_cast<float4*>(p) = v; }
};
template <>
struct Vec4<uint16_t> {
  static __device__ __forceinline__ float4 load(const uint16_t* p) {
    const uint2 u = *reinterpret_cast<const uint2*>(p);
    return make_float4(__uint_as_float(u.x << 16), __uint_as_float(u.x & 0xffff0000u),
                       __uint_as_float(u.y << 16), __uint_as_float(u.y & 0xffff0000u));
  }
  static __device__ __forceinline__ void store(uint16_t* p, float4 v) {
    uint2 u;
    u.x = static_cast<uint32_t>(from_f32<uint16_t>(v.x)) | (static_cast<uint32_t>(from_f32<uint16_t>(v.y)) << 16);
    u.y = static_cast<uint32_t>(from_f32<uint16_t>(v.z)) | (static_cast<uint32_t>(from_f32<uint16_t>(v.w)) << 16);
    *reinterpret_cast<uint2*>(p) = u;
  }
};

// ---------------------------------------------------------------------------
// Cross-lane moves (DPP). quad_bcast<J>: every lane of a quad reads lane J of
// that quad. row_ror<K>: lane i of a 16-lane row reads lane (i + K) mod 16.
// Written as moves; the compiler folds them into the consuming VALU op as a
// DPP source modifier where the encoding allows it.
// ---------------------------------------------------------------------------
template <int J>
__device__ __forceinline__ float quad_bcast(float v) {
  return __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, v), J * 0x55, 0xf, 0xf, true));
}
template <int K>
__device__ __forceinline__ float row_ror(float v) {
  return __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, v), 0x120 + K, 0xf, 0xf, true));
}

// ---------------------------------------------------------------------------
// Chunked selective-scan kernel.
//
// Work: one workgroup per (batch row b, group of 16 consecutive channels).
// It sweeps the sequence in rounds of RT = SEG * TS time steps. Each of the
// SEG waves owns one segment of TS consecutive steps of the round.
//
// Lanes of a wave: lane = 16 r + 4 g + c (r, g, c in 0..3) holds channel
// 4 r + c and the four states n = 4 g .. 4 g + 3 of that channel. The lanes
// of quad g of every row therefore need exactly B_t[4g .. 4g+3] and
// C_t[4g .. 4g+3]: lane q of a row loads B_t[q] and a quad broadcast (DPP)
// hands each lane the other three, without extra VALU work. y_t for a channel
// is the sum over the four quads of a row (two DPP rotate-adds).
//
// Per round:
//   staging  global -> registers (prefetched one round ahead, 16-byte loads)
//            -> LDS tile: (delta, delta*x), D*x, B, C (and, in the forward
//            sweep of the bidirectional scan, the reverse sweep's partial y)
//   local    each wave runs its segment from a zero state, keeping a_t and
//            b_t of all TS steps in registers; segment aggregate
//            (prod a = exp2(A log2e * sum delta), h_end)
//   fold     through LDS: the state entering segment s is the round's carry
//            folded through the aggregates of segments 0..s-1
//   replay   h_t = a_t h_{t-1} + b_t from the true entering state, then the
//            C contraction and the cross-quad sum into the LDS output tile
//   store    the output tile, one round later, 16-byte stores
// With SEG == 1 the carry is known before the segment starts, so the local
// pass is the final pass (no replay).
//
// BIDIR: the same workgroup first sweeps in decreasing time (virtual step
// tau reads time L-1-tau in place, no flipped copy), storing
// sum_n C g + D x as float32 partials, then sweeps forward adding
// sum_n C h to them.
// ---------------------------------------------------------------------------
template <typename T>
struct ScanArgs {
  const T* x;
  const T* dl;
  const float* A;
  const T* B;
  const T* C;
  const float* D;
  T* y;
  float* part;     // bidir: float32 partials of the reverse sweep (may alias y)
  float* h_last;   // forward final state or nullptr
  float* g_first;  // reverse final state or nullptr
  int64_t L;
  int64_t ED;
  int ngroups;     // channel groups per batch row
  int nblocks;
  int remap;       // spread neighbouring channel groups over one XCD
};

template <int RT>
struct alignas(16) Tile {
  float2 xd[RT][16];   // (delta, delta * x) per channel
  float bq[RT][16];    // B_t[n]
  float4 c4[RT][4];    // C_t[4g .. 4g+3]
  float skip[RT][16];  // D * x
  float yt[RT][16];    // sum_n C_t[n] h_t[n] per channel
  float part[RT][16];  // bidir forward sweep: partial from the reverse sweep
};

// Staging of one round: each thread owns TPT fixed (row, chunk) tasks of the
// x/delta tile (4 channels per chunk) or of the B/C tile (4 states per chunk),
// loads them one round ahead into registers, writes them to the LDS tile, and
// stores its chunk of the output tile one round later.
template <typename T, int RT, int TPT>
struct Stager {
  int row[TPT], chk[TPT];
  bool is_xd[TPT];
  float4 dval[TPT];              // D of the chunk's channels
  float4 ra[TPT], rb[TPT], rp[TPT];
  int64_t e0, ED, L;
  bool vec_ok, rev, add_part;

  __device__ __forceinline__ void init(const ScanArgs<T>& p, int tid, int64_t e0_, int64_t ED_) {
    e0 = e0_;
    ED = ED_;
    L = p.L;
    vec_ok = (ED & 3) == 0;
    rev = add_part = false;
#pragma unroll
    for (int k = 0; k < TPT; ++k) {
      int u = tid + k * (8 * RT / TPT);
      is_xd[k] = u < 4 * RT;
      if (!is_xd[k]) u -= 4 * RT;
      row[k] = u >> 2;
      chk[k] = u & 3;
      const int64_t ce = e0 + 4 * chk[k];
      const bool dd = is_xd[k] && p.D != nullptr;
      dval[k] = make_float4(dd && ce + 0 < ED ? p.D[ce + 0] : 0.f, dd && ce + 1 < ED ? p.D[ce + 1] : 0.f,
                            dd && ce + 2 < ED ? p.D[ce + 2] : 0.f, dd && ce + 3 < ED ? p.D[ce + 3] : 0.f);
    }
  }

  __device__ __forceinline__ int64_t time_of(int64_t tau) const { return rev ? (L - 1 - tau) : tau; }

  // global -> registers for round rr
  __device__ __forceinline__ void prefetch(const ScanArgs<T>& p, int64_t b, int64_t rr) {
#pragma unroll
    for (int k = 0; k < TPT; ++k) {
      const int64_t tau = rr * RT + row[k];
      float4 a = make_float4(0.f, 0.f, 0.f, 0.f), bb = a, pp = a;
      if (tau < L) {
        const int64_t t = time_of(tau);
        if (is_xd[k]) {
          const int64_t ce = e0 + 4 * chk[k];
          const int64_t off = (b * L + t) * ED + ce;
          if (vec_ok) {
            if (ce < ED) {
              a = Vec4<T>::load(p.x + off);
              bb = Vec4<T>::load(p.dl + off);
              if (add_part) pp = *reinterpret_cast<const float4*>(p.part + off);
            }
          } else {
            a = make_float4(ce + 0 < ED ? to_f32(p.x[off + 0]) : 0.f, ce + 1 < ED ? to_f32(p.x[off + 1]) : 0.f,
                            ce + 2 < ED ? to_f32(p.x[off + 2]) : 0.f, ce + 3 < ED ? to_f32(p.x[off + 3]) : 0.f);
            bb = make_float4(ce + 0 < ED ? to_f32(p.dl[off + 0]) : 0.f, ce + 1 < ED ? to_f32(p.dl[off + 1]) : 0.f,
                             ce + 2 < ED ? to_f32(p.dl[off + 2]) : 0.f, ce + 3 < ED ? to_f32(p.dl[off + 3]) : 0.f);
            if (add_part)
              pp = make_float4(ce + 0 < ED ? p.part[off + 0] : 0.f, ce + 1 < ED ? p.part[off + 1] : 0.f,
                               ce + 2 < ED ? p.part[off + 2] : 0.f, ce + 3 < ED ? p.part[off + 3] : 0.f);
          }
        } else {
          const int64_t off = (b * L + t) * 16 + 4 * chk[k];
          a = Vec4<T>::load(p.B + off);
          bb = Vec4<T>::load(p.C + off);
        }
      }
      ra[k] = a;
      rb[k] = bb;
      rp[k] = pp;
    }
  }

  // registers -> LDS tile
  __device__ __forceinline__ void commit(Tile<RT>& tl) const {
#pragma unroll
    for (int k = 0; k < TPT; ++k) {
      const int r = row[k], c4 = 4 * chk[k];
      if (is_xd[k]) {
        const float4 xv = ra[k], dv = rb[k];
        *reinterpret_cast<float4*>(&tl.xd[r][c4]) = make_float4(dv.x, dv.x * xv.x, dv.y, dv.y * xv.y);
        *reinterpret_cast<float4*>(&tl.xd[r][c4 + 2]) = make_float4(dv.z, dv.z * xv.z, dv.w, dv.w * xv.w);
        *reinterpret_cast<float4*>(&tl.skip[r][c4]) =
            make_float4(dval[k].x * xv.x, dval[k].y * xv.y, dval[k].z * xv.z, dval[k].w * xv.w);
        if (add_part) *reinterpret_cast<float4*>(&tl.part[r][c4]) = rp[k];
      } else {
        *reinterpret_cast<float4*>(&tl.bq[r][c4]) = ra[k];
        tl.c4[r][chk[k]] = rb[k];
      }
    }
  }

  // LDS output tile of round rr -> global
  __device__ __forceinline__ void store_out(const ScanArgs<T>& p, int64_t b, int64_t rr, const Tile<RT>& tl) const {
#pragma unroll
    for (int k = 0; k < TPT; ++k) {
      if (!is_xd[k]) continue;
      const int r = row[k], c4 = 4 * chk[k];
      const int64_t tau = rr * RT + r;
      const int64_t ce = e0 + c4;
      if (tau >= L || ce >= ED) continue;
      const int64_t off = (b * L + time_of(tau)) * ED + ce;
      const float4 v = *reinterpret_cast<const float4*>(&tl.yt[r][c4]);
      const float4 a = add_part ? *reinterpret_cast<const float4*>(&tl.part[r][c4])
                                : *reinterpret_cast<const float4*>(&tl.skip[r][c4]);
      const float4 o = make_float4(v.x + a.x, v.y + a.y, v.z + a.z, v.w + a.w);
      if (vec_ok) {
        if (rev) *reinterpret_cast<float4*>(p.part + off) = o;
        else Vec4<T>::store(p.y + off, o);
      } else if (rev) {
        p.part[off] = o.x;
        if (ce + 1 < ED) p.part[off + 1] = o.y;
        if (ce + 2 < ED) p.part[off + 2] = o.z;
        if (ce + 3 < ED) p.part[off + 3] = o.w;
      } else {
        p.y[off] = from_f32<T>(o.x);
        if (ce + 1 < ED) p.y[off + 1] = from_f32<T>(o.y);
        if (ce + 2 < ED) p.y[off + 2] = from_f32<T>(o.z);
        if (ce + 3 < ED) p.y[off + 3] = from_f32<T>(o.w);
      }
    }
  }
};

template <typename T, int SEG, int TS, bool BIDIR>
__global__ __launch_bounds__(64 * SEG) void scan_chunked_kernel(const ScanArgs<T> p) {
  constexpr int RT = SEG * TS;
  constexpr int NT = 64 * SEG;
  constexpr int TPT = (8 * RT) / NT;  // staging tasks per thread
  static_assert(TS % 8 == 0, "TS must be a multiple of 8");
  static_assert(TPT * NT == 8 * RT, "staging tasks must divide evenly");

  __shared__ Tile<RT> tile[2];
  __shared__ float4 agg[SEG][64][2];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int q = lane & 15;
  const int g = q >> 2;
  const int ch = ((lane >> 4) << 2) | (q & 3);

  int blk = blockIdx.x;
  if (p.remap) blk = (blk & 7) * (p.nblocks >> 3) + (blk >> 3);
  const int64_t b = blk / p.ngroups;
  const int64_t e0 = static_cast<int64_t>(blk % p.ngroups) * 16;
  const int64_t L = p.L, ED = p.ED;
  const int64_t rounds = (L + RT - 1) / RT;

  // this lane's channel and states
  const int64_t e = e0 + ch;
  const bool ch_ok = e < ED;
  const int64_t ec = ch_ok ? e : ED - 1;
  float A2[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) A2[j] = p.A[ec * 16 + 4 * g + j] * kLog2e;

  Stager<T, RT, TPT> st;
  st.init(p, tid, e0, ED);

  for (int sweep = 0; sweep < (BIDIR ? 2 : 1); ++sweep) {
    const bool rev = BIDIR && sweep == 0;
    const bool add_part = BIDIR && sweep == 1;
    float carry[4] = {0.f, 0.f, 0.f, 0.f};
    st.rev = rev;
    st.add_part = add_part;

    st.prefetch(p, b, 0);
    st.commit(tile[0]);
    __syncthreads();

    for (int64_t r = 0; r < rounds; ++r) {
      Tile<RT>& cur = tile[r & 1];
      Tile<RT>& nxt = tile[(r + 1) & 1];
      if (r + 1 < rounds) st.prefetch(p, b, r + 1);
      if (r >= 1) st.store_out(p, b, r - 1, nxt);

      if constexpr (SEG == 1) {
        // the entering state is known: single pass
#pragma unroll
        for (int i = 0; i < TS; ++i) {
          const float2 xd = cur.xd[i][ch];
          const float bq = cur.bq[i][q];
          const float4 cv = cur.c4[i][g];
          const float bb[4] = {quad_bcast<0>(bq), quad_bcast<1>(bq), quad_bcast<2>(bq), quad_bcast<3>(bq)};
#pragma unroll
          for (int j = 0; j < 4; ++j)
            carry[j] = __builtin_fmaf(__builtin_amdgcn_exp2f(xd.x * A2[j]), carry[j], xd.y * bb[j]);
          float yp = cv.x * carry[0];
          yp = __builtin_fmaf(cv.y, carry[1], yp);
          yp = __builtin_fmaf(cv.z, carry[2], yp);
          yp = __builtin_fmaf(cv.w, carry[3], yp);
          yp += row_ror<4>(yp);
          yp += row_ror<8>(yp);
          if (g == (i & 3)) cur.yt[i][ch] = yp;
        }
      } else {
        // local pass from a zero state
        float av[TS][4], bv[TS][4];
        float hl[4] = {0.f, 0.f, 0.f, 0.f};
        float sd = 0.f;
#pragma unroll
        for (int i = 0; i < TS; ++i) {
          const int row = wave * TS + i;
          const float2 xd = cur.xd[row][ch];
          const float bq = cur.bq[row][q];
          sd += xd.x;
          const float bb[4] = {quad_bcast<0>(bq), quad_bcast<1>(bq), quad_bcast<2>(bq), quad_bcast<3>(bq)};
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            av[i][j] = __builtin_amdgcn_exp2f(xd.x * A2[j]);
            bv[i][j] = xd.y * bb[j];
            hl[j] = __builtin_fmaf(av[i][j], hl[j], bv[i][j]);
          }
        }
        agg[wave][lane][0] = make_float4(__builtin_amdgcn_exp2f(A2[0] * sd), __builtin_amdgcn_exp2f(A2[1] * sd),
                                         __builtin_amdgcn_exp2f(A2[2] * sd), __builtin_amdgcn_exp2f(A2[3] * sd));
        agg[wave][lane][1] = make_float4(hl[0], hl[1], hl[2], hl[3]);
        __syncthreads();

        // fold the segment aggregates in order
        float hin[4] = {carry[0], carry[1], carry[2], carry[3]};
#pragma unroll
        for (int k = 0; k < SEG; ++k) {
          if (k == wave) {
#pragma unroll
            for (int j = 0; j < 4; ++j) hin[j] = carry[j];
          }
          const float4 Ak = agg[k][lane][0], Hk = agg[k][lane][1];
          carry[0] = __builtin_fmaf(Ak.x, carry[0], Hk.x);
          carry[1] = __builtin_fmaf(Ak.y, carry[1], Hk.y);
          carry[2] = __builtin_fmaf(Ak.z, carry[2], Hk.z);
          carry[3] = __builtin_fmaf(Ak.w, carry[3], Hk.w);
        }

        // replay from the entering state
#pragma unroll
        for (int i = 0; i < TS; ++i) {
          const int row = wave * TS + i;
          const float4 cv = cur.c4[row][g];
#pragma unroll
          for (int j = 0; j < 4; ++j) hin[j] = __builtin_fmaf(av[i][j], hin[j], bv[i][j]);
          float yp = cv.x * hin[0];
          yp = __builtin_fmaf(cv.y, hin[1], yp);
          yp = __builtin_fmaf(cv.z, hin[2], yp);
          yp = __builtin_fmaf(cv.w, hin[3], yp);
          yp += row_ror<4>(yp);
          yp += row_ror<8>(yp);
          if (g == (i & 3)) cur.yt[row][ch] = yp;
        }
      }

      if (r + 1 < rounds) st.commit(nxt);
      __syncthreads();
    }
    st.store_out(p, b, rounds - 1, tile[(rounds - 1) & 1]);

    float* h_out = rev ? p.g_first : p.h_last;
    if (h_out && wave == 0 && ch_ok)
      *reinterpret_cast<float4*>(h_out + (b * ED + e) * 16 + 4 * g) = make_float4(carry[0], carry[1], carry[2], carry[3]);
    if (BIDIR) __syncthreads();
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
  const int64_t ngroups = (ED + 15) / 16;
  const int64_t nblk = Bs * ngroups;
  if (nblk > INT32_MAX / 2) return SSM_ERR_DIM;
  ScanArgs<T> a;
  a.x = static_cast<const T*>(x);
  a.dl = static_cast<const T*>(delta);
  a.A = A;
  a.B = static_cast<const T*>(B);
  a.C = static_cast<const T*>(C);
  a.D = D;
  a.y = static_cast<T*>(y);
  a.part = bidir ? (std::is_same<T, float>::value ? reinterpret_cast<float*>(y) : static_cast<float*>(ws)) : nullptr;
  a.h_last = h_last;
  a.g_first = bidir ? g_first : nullptr;
  a.L = L;
  a.ED = ED;
  a.ngroups = static_cast<int>(ngroups);
  a.nblocks = static_cast<int>(nblk);
  a.remap = (nblk % 8 == 0) ? 1 : 0;
  constexpr int SEG = 4, TS = 8;
  if (bidir)
    hipLaunchKernelGGL((scan_chunked_kernel<T, SEG, TS, true>), dim3(nblk), dim3(64 * SEG), 0, stream, a);
  else
    hipLaunchKernelGGL((scan_chunked_kernel<T, SEG, TS, false>), dim3(nblk), dim3(64 * SEG), 0, stream, a);
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
