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

#include <algorithm>
#include <cmath>
#include <cstdint>
#include <atomic>
#include <cstdlib>
#include <cstring>
#include <mutex>
#include <type_traits>

#include "ssm_scan.h"
#include "scan_common.h"

namespace {


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
// C_t[4g .. 4g+3]: lane q of a row reads B_t[q] and C_t[q], and quad
// broadcasts (DPP) hand each lane the other three. Each lane writes its
// partial sum over its four states to LDS; y_t for a channel is the sum of
// the four quads' partials, formed when the output tile is stored.
//
// Per round:
//   staging  global -> registers (prefetched one round ahead, 16-byte loads)
//            -> LDS tile: delta, delta*x, B, C and D*x (in the forward sweep
//            of the bidirectional scan: the reverse sweep's partial y instead)
//   segment  the waves' segments rotate with the round (wave w takes
//            segment (w + round) mod SEG), so that every wave does the same
//            work over SEG rounds
//   first    the wave of segment 0 knows its entering state (the previous
//            round's carry): one pass, h_t = a_t h_{t-1} + b_t, keeping the
//            states; its end state goes to LDS. Its C contraction runs after
//            the round's mid barrier (the store of the previous round reads
//            the output tile before it)
//   local    the other waves run their segments from a zero state, keeping
//            a_t and b_t of all TS steps in registers; segments 1 .. SEG-2
//            also publish their aggregate (prod a = exp2(A log2e * sum
//            delta), h_end) to LDS
//   fold     the state entering segment s > 0 is segment 0's end state
//            folded through the aggregates of segments 1 .. s-1
//   replay   h_t = a_t h_{t-1} + b_t from the true entering state, then the
//            C contraction; the last segment's end state is the round's carry
//   store    one round later: sum of the four state quads + D x (or the
//            reverse sweep's partial), 16-byte stores
// With SEG == 1 the carry is known before the segment starts, so the local
// pass is the final pass (no replay).
//
// BIDIR: the same workgroup first sweeps in decreasing time (virtual step
// tau reads time L-1-tau in place, no flipped copy), storing
// sum_n C g + D x as float32 partials, then sweeps forward adding
// sum_n C h to them.
//
// VEC: ED is a multiple of 4, so every 4-channel chunk is 16-byte (float32)
// or 8-byte (bfloat16) aligned and either wholly inside or wholly outside
// [0, ED); otherwise chunks are loaded and stored element by element.
// ---------------------------------------------------------------------------
// Cross-workgroup state of the split-sequence scan (device workspace). A
// sequence too long for the available channel parallelism is cut into
// chunks that run concurrently; chunk k hands its inclusive end state to
// chunk k+1 through `state` and `flag`.
//
// Protocol. The chunks are dealt out through 8 ticket queues, one per XCD:
// queue q holds the chunks of a contiguous range of channel groups, chunk-
// major (chunk 0 of each of its groups, then chunk 1, ...). A workgroup
// takes a ticket from the queue of the XCD it runs on (so that neighbouring
// groups, which share 128-byte lines of x, delta and y, are served by one
// L2), and only if that queue is exhausted from the next ones in turn. Every
// queue is consumed in ticket order and a chunk's predecessor sits in the
// same queue at an earlier ticket, so it has already started, whichever
// workgroups the hardware dispatches first and to which XCD, and whatever
// else runs on the device; there are as many workgroups as chunks, so every
// chunk is taken. A started chunk finishes its main pass without waiting on
// anything, then (chunk k > 0) waits for flag[k-1], reads state[k-1]
// (acquire), publishes its own inclusive state and raises flag[k] (release);
// a chunk's wait therefore only depends on earlier tickets, and every wait
// ends. The wait is still bounded (a few seconds): if it ever gives up, `err`
// is set and the chunk takes NaN as its entering state, so that its outputs,
// its published state and every later chunk's become NaN rather than silently
// wrong; ssm_scan_fwd_status() reports the error word to the host.
constexpr int kQueues = 8;
struct SplitHeader {
  unsigned err;              // nonzero: a wait gave up (never expected)
  unsigned ticket[kQueues];  // next ticket of each queue
  unsigned pad[64 - 1 - kQueues];
};

template <typename T>
struct ScanArgs {
  const T* x;
  const T* dl;
  const float* A;
  const T* B;
  const T* C;
  const float* D;
  const float* h0;  // initial forward state (Bs, ED, N) or nullptr for zero
  const float* g0;  // bidirectional: reverse state entering at t = L-1 (Bs, ED, N), or nullptr for zero
  // step-size pre-processing: delta' = clamp(softplus?(delta + dt_bias), dt_min, dt_max)
  const float* dt_bias;  // (ED) or nullptr
  int dt_softplus;
  int dt_pre;            // any pre-processing at all
  float dt_min, dt_max;
  const T* z;            // gate (Bs, L, ED): y *= z sigmoid(z); used when GATE
  T* y;
  float* part;     // bidir: float32 partials of the reverse sweep (may alias y)
  float* h_last;   // forward final state or nullptr
  float* g_first;  // reverse final state or nullptr
  int64_t L;
  int64_t ED;
  int ngroups;     // channel groups per batch row
  int nblocks;
  int remap;       // spread neighbouring channel groups over one XCD
  int rot_ncu;     // compute units, when every workgroup is resident at once; else 0 (no priority rotation)
  // split sequence (nchunks > 1)
  int nchunks;
  int64_t chunk_len;    // multiple of the round length
  unsigned spin_limit;  // iterations of a hand-off wait before it gives up
  SplitHeader* hdr;
  int* flag;            // [bg * nchunks + k]
  float* state;         // [bg * nchunks + k][16 channels][16 states]
  // bidirectional split: per chunk, the sum of delta per channel and the
  // reverse sweep's start state (state: the forward sweep's end state)
  double* sdsum;        // [bg * nchunks + k][16 channels]
  float* gstate;        // [bg * nchunks + k][16 channels][16 states]
  // round checkpoints (forward scans only, or nullptr): the state entering
  // every round of kRT steps, [Bs][ck_rounds][ck_EDp][16], round 0 not written
  float* ckpt;
  int64_t ck_rounds, ck_EDp;
};

// Input tile of one round (double-buffered).
template <int RT, bool GATE>
struct alignas(16) Tile {
  float dt[RT][16];   // delta per channel
  float dx[RT][16];   // delta * x per channel
  float bq[RT][16];   // B_t[n]
  float cq[RT][16];   // C_t[n]
  float aux[RT][16];  // D x; the reverse sweep's partial (bidir forward sweep); y so far (correction pass)
  float gate[GATE ? RT : 1][16];  // z sigmoid(z)
};

// Output tile of one round (single-buffered: written by the replay after the
// round's mid barrier, read by the store at the start of the next round).
template <int RT>
struct alignas(16) OutTile {
  float yq[4][RT + 1][16];  // per state quad g: sum over its 4 states of C h (rows padded)
};

// Segment aggregates and the carry between rounds.
template <int SEG, bool SPLIT>
struct alignas(16) FoldArea {
  float4 A[SEG][64];    // prod of a over the segment, per lane's 4 states
  float4 H[SEG][64];    // state at the segment's end, started from zero
  float4 carry[2][64];  // state after the round, by round parity
  double sd[SPLIT ? SEG : 1][64];  // split sequence: sum of delta over each wave's segments
};

enum { STAGE_SCAN = 0, STAGE_CORRECT = 1 };

// The split sequence's correction pass drops a carried term once its decay
// product is below 2^-kCorrectionCut: what it leaves out is 2^6 below the
// float32 rounding of the sum it would be added to.
constexpr float kCorrectionCut = 30.f;

// delta' = clamp(softplus?(delta + dt_bias[e]), dt_min, dt_max), with the
// channel's bias (0 without one) already in a register
template <typename T>
__device__ __forceinline__ float step_size(const ScanArgs<T>& p, float d, float bias) {
  return map_step(d + bias, nullptr, p.dt_softplus, p.dt_min, p.dt_max);
}

// Staging of one round: each thread owns TPT fixed (row, chunk) tasks of the
// x/delta tile (4 channels per chunk) or of the B/C tile (4 states per chunk),
// loads them one round ahead into registers, writes them to the LDS tile, and
// stores its chunk of the output tile one round later. Offsets advance by one
// round (RT steps, forward or backward in time) per call. A pass covers the
// Lk steps starting at time t0 (the whole sequence unless it is split).
template <typename T, int RT, int TPT, bool BIDIR, bool VEC, bool GATE>
struct Stager {
  int row[TPT], chk[TPT];
  bool is_xd[TPT], chunk_ok[TPT], row_ok[TPT];
  float4 dval[TPT];              // D of the chunk's channels
  float4 bval[TPT];              // dt_bias of the chunk's channels (0 without a bias), loaded once
  // prefetched data: loaded bits (VEC; widened at commit, so that the wave
  // does not wait for the loads at the prefetch), or widened values (element
  // by element loads of a ragged channel count)
  typename Vec4<T>::Raw qa[VEC ? TPT : 1], qb[VEC ? TPT : 1], qy[VEC ? TPT : 1], qz[VEC ? TPT : 1];
  float4 qp[VEC ? TPT : 1];      // the reverse sweep's float32 partial
  bool ld_ok[TPT];
  float4 ra[TPT], rb[TPT], rp[TPT], rz[TPT];
  int64_t pre_off[TPT];          // element offset of this task's row in the next round to prefetch
  int64_t out_off[TPT];          // element offset of this task's row in the next round to store
  int64_t step_xd, step_bc;      // offset change per round
  int64_t ce0;                   // first channel of the group
  int64_t ED, Lk;
  bool rev, add_part;

  __device__ __forceinline__ void init(const ScanArgs<T>& p, int tid, int64_t e0) {
    ED = p.ED;
    ce0 = e0;
#pragma unroll
    for (int k = 0; k < TPT; ++k) {
      int u = tid + k * (8 * RT / TPT);
      is_xd[k] = u < 4 * RT;
      if (!is_xd[k]) u -= 4 * RT;
      row[k] = u >> 2;
      chk[k] = u & 3;
      const int64_t ce = e0 + 4 * chk[k];
      chunk_ok[k] = !is_xd[k] || ce < ED;
      const bool dd = is_xd[k] && p.D != nullptr;
      dval[k] = make_float4(dd && ce + 0 < ED ? p.D[ce + 0] : 0.f, dd && ce + 1 < ED ? p.D[ce + 1] : 0.f,
                            dd && ce + 2 < ED ? p.D[ce + 2] : 0.f, dd && ce + 3 < ED ? p.D[ce + 3] : 0.f);
      const bool db = is_xd[k] && p.dt_bias != nullptr;
      bval[k] = make_float4(db && ce + 0 < ED ? p.dt_bias[ce + 0] : 0.f, db && ce + 1 < ED ? p.dt_bias[ce + 1] : 0.f,
                            db && ce + 2 < ED ? p.dt_bias[ce + 2] : 0.f, db && ce + 3 < ED ? p.dt_bias[ce + 3] : 0.f);
    }
  }

  // start a pass over times [t0, t0 + Lk) (reverse: t0 + Lk - 1 down to t0)
  __device__ __forceinline__ void begin(int64_t b, int64_t L, int64_t t0, int64_t Lk_, bool rev_, bool add_part_) {
    Lk = Lk_;
    rev = rev_;
    add_part = add_part_;
    step_xd = (rev ? -RT : RT) * ED;
    step_bc = (rev ? -RT : RT) * 16;
#pragma unroll
    for (int k = 0; k < TPT; ++k) {
      const int64_t t = rev ? (t0 + Lk - 1 - row[k]) : (t0 + row[k]);
      pre_off[k] = is_xd[k] ? (b * L + t) * ED + ce0 + 4 * chk[k] : (b * L + t) * 16 + 4 * chk[k];
      out_off[k] = pre_off[k];
    }
  }

  // global -> registers for round rr. STAGE_SCAN: x, delta, B, C (and the
  // reverse sweep's partial); STAGE_CORRECT: delta, C and the current y.
  template <int STAGE>
  __device__ __forceinline__ void prefetch(const ScanArgs<T>& p, int64_t rr) {
#pragma unroll
    for (int k = 0; k < TPT; ++k) {
      const int64_t off = pre_off[k];
      pre_off[k] += is_xd[k] ? step_xd : step_bc;
      row_ok[k] = rr * RT + row[k] < Lk;
      ld_ok[k] = row_ok[k] && chunk_ok[k];
      if constexpr (VEC) {
        // rows past the end read element 0 instead (in bounds); commit drops them
        const int64_t lo = ld_ok[k] ? off : 0;
        if (!is_xd[k]) {
          if (STAGE == STAGE_SCAN) qa[k] = Vec4<T>::load_raw(p.B + lo);
          qb[k] = Vec4<T>::load_raw(p.C + lo);
        } else {
          if (STAGE == STAGE_SCAN) qa[k] = Vec4<T>::load_raw(p.x + lo);
          qb[k] = Vec4<T>::load_raw(p.dl + lo);
          if (STAGE == STAGE_CORRECT) qy[k] = Vec4<T>::load_raw(p.y + lo);
          if (BIDIR && add_part) qp[k] = *reinterpret_cast<const float4*>(p.part + lo);
          if (GATE) qz[k] = Vec4<T>::load_raw(p.z + lo);
        }
        continue;
      }
      float4 a = make_float4(0.f, 0.f, 0.f, 0.f), bb = a, pp = a, zz = a;
      if (row_ok[k] && chunk_ok[k]) {
        if (!is_xd[k]) {
          if (STAGE == STAGE_SCAN) a = Vec4<T>::load(p.B + off);
          bb = Vec4<T>::load(p.C + off);
        } else {
          const int64_t ce = ce0 + 4 * chk[k];
          if (STAGE == STAGE_SCAN)
            a = make_float4(to_f32(p.x[off]), ce + 1 < ED ? to_f32(p.x[off + 1]) : 0.f,
                            ce + 2 < ED ? to_f32(p.x[off + 2]) : 0.f, ce + 3 < ED ? to_f32(p.x[off + 3]) : 0.f);
          bb = make_float4(to_f32(p.dl[off]), ce + 1 < ED ? to_f32(p.dl[off + 1]) : 0.f,
                           ce + 2 < ED ? to_f32(p.dl[off + 2]) : 0.f, ce + 3 < ED ? to_f32(p.dl[off + 3]) : 0.f);
          if (STAGE == STAGE_CORRECT)
            pp = make_float4(to_f32(p.y[off]), ce + 1 < ED ? to_f32(p.y[off + 1]) : 0.f,
                             ce + 2 < ED ? to_f32(p.y[off + 2]) : 0.f, ce + 3 < ED ? to_f32(p.y[off + 3]) : 0.f);
          if (BIDIR && add_part)
            pp = make_float4(p.part[off], ce + 1 < ED ? p.part[off + 1] : 0.f, ce + 2 < ED ? p.part[off + 2] : 0.f,
                             ce + 3 < ED ? p.part[off + 3] : 0.f);
          if (GATE)
            zz = make_float4(to_f32(p.z[off]), ce + 1 < ED ? to_f32(p.z[off + 1]) : 0.f,
                             ce + 2 < ED ? to_f32(p.z[off + 2]) : 0.f, ce + 3 < ED ? to_f32(p.z[off + 3]) : 0.f);
        }
      }
      ra[k] = a;
      rb[k] = bb;
      rp[k] = pp;
      if (GATE) rz[k] = zz;
    }
  }

  // prefetched values of task k (zero for rows past the end)
  __device__ __forceinline__ float4 val_a(int k) const {
    if constexpr (VEC) return ld_ok[k] ? Vec4<T>::widen(qa[k]) : make_float4(0.f, 0.f, 0.f, 0.f);
    return ra[k];
  }
  __device__ __forceinline__ float4 val_b(int k) const {
    if constexpr (VEC) return ld_ok[k] ? Vec4<T>::widen(qb[k]) : make_float4(0.f, 0.f, 0.f, 0.f);
    return rb[k];
  }
  template <int STAGE>
  __device__ __forceinline__ float4 val_p(int k) const {
    if constexpr (VEC) {
      const float4 z4 = make_float4(0.f, 0.f, 0.f, 0.f);
      if (STAGE == STAGE_CORRECT) return ld_ok[k] ? Vec4<T>::widen(qy[k]) : z4;
      return ld_ok[k] ? qp[k] : z4;
    }
    return rp[k];
  }
  __device__ __forceinline__ float4 val_z(int k) const {
    if constexpr (VEC) return ld_ok[k] ? Vec4<T>::widen(qz[k]) : make_float4(0.f, 0.f, 0.f, 0.f);
    return rz[k];
  }

  // registers -> LDS tile
  template <int STAGE>
  __device__ __forceinline__ void commit(const ScanArgs<T>& p, Tile<RT, GATE>& tl) const {
#pragma unroll
    for (int k = 0; k < TPT; ++k) {
      const int r = row[k], c4 = 4 * chk[k];
      if (is_xd[k]) {
        const float4 xv = val_a(k);
        float4 dv = val_b(k);
        if (p.dt_pre) {
          // padded rows and channels keep delta = 0 (a = 1, b = 0: no effect)
          const bool ok = row_ok[k] && chunk_ok[k];
          const int64_t ce = ce0 + c4;
          dv.x = ok && ce + 0 < ED ? step_size(p, dv.x, bval[k].x) : 0.f;
          dv.y = ok && ce + 1 < ED ? step_size(p, dv.y, bval[k].y) : 0.f;
          dv.z = ok && ce + 2 < ED ? step_size(p, dv.z, bval[k].z) : 0.f;
          dv.w = ok && ce + 3 < ED ? step_size(p, dv.w, bval[k].w) : 0.f;
        }
        if (GATE) {
          const float4 zv = val_z(k);
          *reinterpret_cast<float4*>(&tl.gate[r][c4]) = make_float4(silu(zv.x), silu(zv.y), silu(zv.z), silu(zv.w));
        }
        *reinterpret_cast<float4*>(&tl.dt[r][c4]) = dv;
        if (STAGE == STAGE_CORRECT) {
          *reinterpret_cast<float4*>(&tl.aux[r][c4]) = val_p<STAGE>(k);
        } else {
          *reinterpret_cast<float4*>(&tl.dx[r][c4]) =
              make_float4(dv.x * xv.x, dv.y * xv.y, dv.z * xv.z, dv.w * xv.w);
          *reinterpret_cast<float4*>(&tl.aux[r][c4]) =
              (BIDIR && add_part)
                  ? val_p<STAGE>(k)
                  : make_float4(dval[k].x * xv.x, dval[k].y * xv.y, dval[k].z * xv.z, dval[k].w * xv.w);
        }
      } else {
        if (STAGE == STAGE_SCAN) *reinterpret_cast<float4*>(&tl.bq[r][c4]) = val_a(k);
        *reinterpret_cast<float4*>(&tl.cq[r][c4]) = val_b(k);
      }
    }
  }

  // output of round rr (whose input tile is tl) -> global:
  //   scan pass:       (sum over the state quads + aux) * gate
  //   reverse sweep:   sum + aux (float32 partial, no gate)
  //   correction pass: aux + sum * gate
  template <int STAGE>
  __device__ __forceinline__ void store_out(const ScanArgs<T>& p, int64_t rr, const Tile<RT, GATE>& tl,
                                            const OutTile<RT>& ot) {
#pragma unroll
    for (int k = 0; k < TPT; ++k) {
      if (!is_xd[k]) continue;
      const int64_t off = out_off[k];
      out_off[k] += step_xd;
      const int r = row[k], c4 = 4 * chk[k];
      if (rr * RT + r >= Lk || !chunk_ok[k]) continue;
      const float4 v0 = *reinterpret_cast<const float4*>(&ot.yq[0][r][c4]);
      const float4 v1 = *reinterpret_cast<const float4*>(&ot.yq[1][r][c4]);
      const float4 v2 = *reinterpret_cast<const float4*>(&ot.yq[2][r][c4]);
      const float4 v3 = *reinterpret_cast<const float4*>(&ot.yq[3][r][c4]);
      const float4 a = *reinterpret_cast<const float4*>(&tl.aux[r][c4]);
      float4 o = make_float4((v0.x + v1.x) + (v2.x + v3.x), (v0.y + v1.y) + (v2.y + v3.y),
                             (v0.z + v1.z) + (v2.z + v3.z), (v0.w + v1.w) + (v2.w + v3.w));
      if (STAGE == STAGE_SCAN) o = make_float4(o.x + a.x, o.y + a.y, o.z + a.z, o.w + a.w);
      if (GATE && !(BIDIR && rev)) {
        const float4 gv = *reinterpret_cast<const float4*>(&tl.gate[r][c4]);
        o = make_float4(o.x * gv.x, o.y * gv.y, o.z * gv.z, o.w * gv.w);
      }
      if (STAGE == STAGE_CORRECT) o = make_float4(a.x + o.x, a.y + o.y, a.z + o.z, a.w + o.w);
      if (VEC) {
        if (BIDIR && rev) *reinterpret_cast<float4*>(p.part + off) = o;
        else Vec4<T>::store(p.y + off, o);
      } else {
        const int64_t ce = ce0 + c4;
        if (BIDIR && rev) {
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
  }
};

// Wait, bounded, until another workgroup sets *flag; called by one lane.
// Returns false (and sets *err) if the wait gave up.
__device__ __forceinline__ bool wait_flag(int* flag, unsigned* err, unsigned spin_limit) {
  for (unsigned it = 0;; ++it) {
    if (__hip_atomic_load(flag, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) != 0) return true;
    if (it >= spin_limit) {  // ~ seconds at the default limit: give up rather than hang the device
      __hip_atomic_fetch_or(err, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      return false;
    }
    __builtin_amdgcn_s_sleep(4);
  }
}

// Queue q of the split-sequence chunks holds the groups [q nbg / 8,
// (q + 1) nbg / 8), each in nchunks chunks, chunk-major.
__device__ __forceinline__ int split_queue_start(int q, int nbg) { return q * nbg / kQueues; }

// Takes a chunk for this workgroup (thread 0): a ticket from the queue of the
// XCD it runs on, else from the following queues in turn. Returns the chunk
// index and channel group, or false if every queue is exhausted (impossible
// with one workgroup per chunk).
__device__ __forceinline__ bool split_take_chunk(unsigned* tickets, int nbg, int nchunks, int64_t* kchunk,
                                                 int64_t* bg) {
  // XCC_ID hardware register (bits 3:0): the XCD this wave runs on
  const unsigned xcc = static_cast<unsigned>(__builtin_amdgcn_s_getreg((3 << 11) | (0 << 6) | 20));
  for (int d = 0; d < kQueues; ++d) {
    const int q = static_cast<int>((xcc + d) % kQueues);
    const int g0 = split_queue_start(q, nbg), ng = split_queue_start(q + 1, nbg) - g0;
    if (ng == 0) continue;
    const unsigned j = __hip_atomic_fetch_add(&tickets[q], 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    if (j < static_cast<unsigned>(ng * nchunks)) {
      *kchunk = j / ng;
      *bg = g0 + static_cast<int>(j % ng);
      return true;
    }
  }
  return false;
}

// ---- correction of a chunk's outputs for the state entering it ----------
// Forward (rev = false): y_t += sum_n C_t[n] (prod_{s = t0 .. t} a_s[n]) h_in[n]
// from the chunk's first step on; reverse (rev = true): the same with the
// product over s = t .. t_end and the state entering at the chunk's last
// step, from that step backwards. The product is exp2(A log2e * cumulative
// delta) (a float64 running sum). With delta >= 0 and A <= 0 (checked as we
// go) the products only decay; once every one is below 2^-kCorrectionCut (or
// its h_in is zero) the pass stops. The terms it leaves out add at most
// 2^-kCorrectionCut sum_n |C_t[n] h_in[n]| to any y_t, far below one float32
// rounding of that sum. A poisoned (NaN) h_in is carried to the chunk's end.
// The output gate, if any, multiplies the correction.
template <typename T, int SEG, int TS, bool VEC, bool GATE, int TPT>
__device__ void correct_pass(const ScanArgs<T>& p, Stager<T, SEG * TS, TPT, false, VEC, GATE>& st,
                             Tile<SEG * TS, GATE> (&tile)[2], OutTile<SEG * TS>& out, int64_t b, int64_t t0,
                             int64_t Lk, bool rev, const float (&hin)[4], const float (&A2)[4], int wave, int ch,
                             int q, int g) {
  constexpr int RT = SEG * TS;
  const int64_t rounds = (Lk + RT - 1) / RT;
  bool mono = A2[0] <= 0.f && A2[1] <= 0.f && A2[2] <= 0.f && A2[3] <= 0.f;
  const bool poisoned = hin[0] != hin[0] || hin[1] != hin[1] || hin[2] != hin[2] || hin[3] != hin[3];
  double base = 0.0;  // cumulative delta before the current round
  st.begin(b, p.L, t0, Lk, rev, false);
  st.template prefetch<STAGE_CORRECT>(p, 0);
  st.template commit<STAGE_CORRECT>(p, tile[0]);
  __syncthreads();
  for (int64_t r = 0; r < rounds; ++r) {
    Tile<RT, GATE>& cur = tile[r & 1];
    Tile<RT, GATE>& nxt = tile[(r + 1) & 1];
    if (r + 1 < rounds) st.template prefetch<STAGE_CORRECT>(p, r + 1);
    if (r >= 1) st.template store_out<STAGE_CORRECT>(p, r - 1, nxt, out);
    if (p.ckpt && !rev && wave == 0) {
      // the checkpoint of this round: the main pass's state (from zero at the
      // chunk's start) plus the entering state carried to the round's start;
      // the chunk's first round is the entering state itself
      float* ck = p.ckpt + ((b * p.ck_rounds + t0 / RT + r) * p.ck_EDp + st.ce0 + ch) * 16 + 4 * g;
      float4 v = r == 0 ? make_float4(0.f, 0.f, 0.f, 0.f) : *reinterpret_cast<const float4*>(ck);
      const float cb = static_cast<float>(base);
      v.x = __builtin_fmaf(__builtin_amdgcn_exp2f(A2[0] * cb), hin[0], v.x);
      v.y = __builtin_fmaf(__builtin_amdgcn_exp2f(A2[1] * cb), hin[1], v.y);
      v.z = __builtin_fmaf(__builtin_amdgcn_exp2f(A2[2] * cb), hin[2], v.z);
      v.w = __builtin_fmaf(__builtin_amdgcn_exp2f(A2[3] * cb), hin[3], v.w);
      *reinterpret_cast<float4*>(ck) = v;
    }
    __syncthreads();  // the output tile is reused below
    float pre = 0.f;  // delta of the round's rows before this wave's segment
    for (int i = 0; i < wave * TS; ++i) pre += cur.dt[i][ch];
    bool alive = false;
#pragma unroll
    for (int i = 0; i < TS; ++i) {
      const int row = wave * TS + i;
      const float dt = cur.dt[row][ch];
      mono = mono && dt >= 0.f;
      pre += dt;
      const float cum = static_cast<float>(base + static_cast<double>(pre));
      float w[4];
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const float e2 = A2[j] * cum;
        w[j] = __builtin_amdgcn_exp2f(e2) * hin[j];
        alive = alive || (e2 > -kCorrectionCut && hin[j] != 0.f);
      }
      const float cq = cur.cq[row][q];
      const float yp = dot_quad(cq, w);
      out.yq[g][row][ch] = yp;
    }
    float rest = 0.f;  // rows after this wave's segment
    for (int i = (wave + 1) * TS; i < RT; ++i) rest += cur.dt[i][ch];
    base += static_cast<double>(pre + rest);
    if (r + 1 < rounds) st.template commit<STAGE_CORRECT>(p, nxt);
    const int go_on = __syncthreads_or((alive || !mono || poisoned) ? 1 : 0);
    if (!go_on) {
      st.template store_out<STAGE_CORRECT>(p, r, cur, out);
      return;
    }
  }
  st.template store_out<STAGE_CORRECT>(p, rounds - 1, tile[(rounds - 1) & 1], out);
}

template <typename T, int SEG, int TS, bool BIDIR, bool VEC, bool SPLIT, bool GATE, int WPE = 3>
__global__ __launch_bounds__(64 * SEG) __attribute__((amdgpu_waves_per_eu(WPE))) void scan_chunked_kernel(
    const ScanArgs<T> p) {
  constexpr int RT = SEG * TS;
  constexpr int NT = 64 * SEG;
  constexpr int TPT = (8 * RT) / NT;  // staging tasks per thread
  static_assert(TS % 8 == 0, "TS must be a multiple of 8");
  static_assert(TPT * NT == 8 * RT, "staging tasks must divide evenly");
  static_assert(!SPLIT || SEG > 1, "the split-sequence scan needs several segments");

  __shared__ Tile<RT, GATE> tile[2];
  __shared__ OutTile<RT> out;
  __shared__ FoldArea<SEG, SPLIT> fa;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int q = lane & 15;
  const int g = q >> 2;
  const int ch = ((lane >> 4) << 2) | (q & 3);
  const int64_t L = p.L, ED = p.ED;

  // which (batch row, channel group) and, for a split sequence, which chunk.
  // Consecutive logical blocks share an XCD (its L2 serves the cache lines
  // that neighbouring channel groups share). A split sequence takes its chunk
  // from a per-XCD ticket queue (see SplitHeader): a chunk's predecessor holds
  // an earlier ticket of the same queue, so it has started and its state will
  // be published.
  int64_t bg, kchunk = 0, t0 = 0, Lk = L;
  if constexpr (SPLIT && BIDIR) {
    // the bidirectional split waits for nothing (a second kernel joins the
    // chunks), so its chunks follow the block index, chunk-major
    int64_t blk = blockIdx.x;
    if (p.remap) blk = (blk & 7) * (p.nblocks >> 3) + (blk >> 3);
    const int64_t nbg = p.nblocks / p.nchunks;
    kchunk = blk / nbg;
    bg = blk % nbg;
    t0 = kchunk * p.chunk_len;
    Lk = L - t0 < p.chunk_len ? L - t0 : p.chunk_len;
  } else if constexpr (SPLIT) {
    __shared__ int s_chunk[2];
    if (tid == 0) {
      int64_t k = 0, g = 0;
      if (split_take_chunk(p.hdr->ticket, p.nblocks / p.nchunks, p.nchunks, &k, &g)) {
        s_chunk[0] = static_cast<int>(k);
        s_chunk[1] = static_cast<int>(g);
      } else {
        s_chunk[0] = -1;
        __hip_atomic_fetch_or(&p.hdr->err, 2u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      }
    }
    __syncthreads();
    if (s_chunk[0] < 0) return;  // (uniform; cannot happen: as many workgroups as chunks)
    kchunk = s_chunk[0];
    bg = s_chunk[1];
    t0 = kchunk * p.chunk_len;
    Lk = L - t0 < p.chunk_len ? L - t0 : p.chunk_len;
  } else {
    int blk = blockIdx.x;
    if (p.remap) blk = (blk & 7) * (p.nblocks >> 3) + (blk >> 3);
    bg = blk;
  }
  const int64_t b = bg / p.ngroups;
  const int64_t e0 = (bg % p.ngroups) * 16;
  const int64_t rounds = (Lk + RT - 1) / RT;

  // this lane's channel and states
  const int64_t e = e0 + ch;
  const bool ch_ok = e < ED;
  const int64_t ec = ch_ok ? e : ED - 1;
  float A2[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) A2[j] = p.A[ec * 16 + 4 * g + j] * kLog2e;

  Stager<T, RT, TPT, BIDIR, VEC, GATE> st;
  st.init(p, tid, e0);
  double sd_total = 0.0;  // split sequence: sum of delta over this wave's segments (of the last sweep)
  float carry[4];         // state after the last completed round (valid in wave SEG-1 after the sweep)
  float gloc[4] = {0.f, 0.f, 0.f, 0.f};  // bidirectional split: the reverse sweep's end state

  for (int sweep = 0; sweep < (BIDIR ? 2 : 1); ++sweep) {
    const bool rev = BIDIR && sweep == 0;
    st.begin(b, L, t0, Lk, rev, BIDIR && sweep == 1);
    sd_total = 0.0;
    // entering state: h0 for the forward sweep's first chunk, g0 for the
    // reverse sweep's first (the sequence's last) chunk, else zero
    float4 init = make_float4(0.f, 0.f, 0.f, 0.f);
    if (p.h0 && !rev && kchunk == 0 && ch_ok) init = *reinterpret_cast<const float4*>(p.h0 + (b * ED + e) * 16 + 4 * g);
    if (BIDIR && p.g0 && rev && kchunk == p.nchunks - 1 && ch_ok)
      init = *reinterpret_cast<const float4*>(p.g0 + (b * ED + e) * 16 + 4 * g);
    carry[0] = init.x, carry[1] = init.y, carry[2] = init.z, carry[3] = init.w;
    if (SEG > 1 && wave == SEG - 1) fa.carry[1][lane] = init;

    st.template prefetch<STAGE_SCAN>(p, 0);
    st.template commit<STAGE_SCAN>(p, tile[0]);
    __syncthreads();

    for (int64_t r = 0; r < rounds; ++r) {
      Tile<RT, GATE>& cur = tile[r & 1];
      Tile<RT, GATE>& nxt = tile[(r + 1) & 1];
      rotate_priority(r, p.rot_ncu);
      if (r + 1 < rounds) st.template prefetch<STAGE_SCAN>(p, r + 1);
      // output of round r-1, whose input tile stays intact until this round's commit
      if (r >= 1) st.template store_out<STAGE_SCAN>(p, r - 1, nxt, out);

      if constexpr (SEG == 1) {
        // the output tile is single-buffered: the store above must finish
        // reading it before this round writes it
        __syncthreads();
        // the entering state is known: single pass
#pragma unroll
        for (int i = 0; i < TS; ++i) {
          const float dt = cur.dt[i][ch], dx = cur.dx[i][ch];
          const float bq = cur.bq[i][q], cq = cur.cq[i][q];
          const float bb[4] = {quad_bcast<0>(bq), quad_bcast<1>(bq), quad_bcast<2>(bq), quad_bcast<3>(bq)};
#pragma unroll
          for (int j = 0; j < 4; ++j)
            carry[j] = __builtin_fmaf(__builtin_amdgcn_exp2f(dt * A2[j]), carry[j], dx * bb[j]);
          const float yp = dot_quad(cq, carry);
          out.yq[g][i][ch] = yp;
        }
      } else {
        // This wave's segment of the round. The roles rotate with the round,
        // so that over SEG rounds every wave (and SIMD) does the same work.
        const int seg = (wave + static_cast<int>(r)) & (SEG - 1);
        float av[TS][4], bv[TS][4];
        if (seg == 0) {
          // the entering state is the previous round's carry: a single pass,
          // whose end state is the exact state entering segment 1
          const float4 c0 = fa.carry[(r + 1) & 1][lane];
          float h[4] = {c0.x, c0.y, c0.z, c0.w};
          float sd = 0.f;
#pragma unroll
          for (int i = 0; i < TS; ++i) {
            const float dt = cur.dt[i][ch], dx = cur.dx[i][ch];
            const float bq = cur.bq[i][q];
            if (SPLIT) sd += dt;
            const float bb[4] = {quad_bcast<0>(bq), quad_bcast<1>(bq), quad_bcast<2>(bq), quad_bcast<3>(bq)};
#pragma unroll
            for (int j = 0; j < 4; ++j) {
              // (a_t and b_t go to av / bv like the other segments' values, so
              // that both paths leave them in the same registers; once used,
              // av keeps the state h_t for the contraction after the barrier)
              av[i][j] = __builtin_amdgcn_exp2f(dt * A2[j]);
              bv[i][j] = dx * bb[j];
              h[j] = __builtin_fmaf(av[i][j], h[j], bv[i][j]);
              av[i][j] = h[j];
            }
          }
          if (SPLIT) sd_total += static_cast<double>(sd);
          fa.H[0][lane] = make_float4(h[0], h[1], h[2], h[3]);
        } else {
          // local pass from a zero state: a_t and b_t of every step
          float sd = 0.f;
#pragma unroll
          for (int i = 0; i < TS; ++i) {
            const int row = seg * TS + i;
            const float dt = cur.dt[row][ch], dx = cur.dx[row][ch];
            const float bq = cur.bq[row][q];
            sd += dt;
            const float bb[4] = {quad_bcast<0>(bq), quad_bcast<1>(bq), quad_bcast<2>(bq), quad_bcast<3>(bq)};
#pragma unroll
            for (int j = 0; j < 4; ++j) {
              av[i][j] = __builtin_amdgcn_exp2f(dt * A2[j]);
              bv[i][j] = dx * bb[j];
            }
          }
          if (SPLIT) sd_total += static_cast<double>(sd);
          if (seg < SEG - 1) {
            // aggregate for the later segments (the last one needs none):
            // prod a = exp2(A log2e * sum delta) and the end state from zero
            float hl[4] = {bv[0][0], bv[0][1], bv[0][2], bv[0][3]};
#pragma unroll
            for (int i = 1; i < TS; ++i)
#pragma unroll
              for (int j = 0; j < 4; ++j) hl[j] = __builtin_fmaf(av[i][j], hl[j], bv[i][j]);
            fa.A[seg][lane] = make_float4(__builtin_amdgcn_exp2f(A2[0] * sd), __builtin_amdgcn_exp2f(A2[1] * sd),
                                          __builtin_amdgcn_exp2f(A2[2] * sd), __builtin_amdgcn_exp2f(A2[3] * sd));
            fa.H[seg][lane] = make_float4(hl[0], hl[1], hl[2], hl[3]);
          }
        }
        __syncthreads();

        if (seg == 0) {
          // the C contraction of segment 0's states; the output tile may be
          // read by this round's store of the previous round until the barrier.
          // (Doing it here also balances the two phases' work over the waves.)
#pragma unroll
          for (int i = 0; i < TS; ++i) out.yq[g][i][ch] = dot_quad(cur.cq[i][q], av[i]);
        } else {
          // entering state: segment 0's end state through segments 1 .. seg-1
          // (seg is uniform, so the loop bound is scalar)
          const float4 c0 = fa.H[0][lane];
          float hin[4] = {c0.x, c0.y, c0.z, c0.w};
#pragma unroll 1
          for (int k = 1; k < seg; ++k) {
            const float4 Ak = fa.A[k][lane], Hk = fa.H[k][lane];
            hin[0] = __builtin_fmaf(Ak.x, hin[0], Hk.x);
            hin[1] = __builtin_fmaf(Ak.y, hin[1], Hk.y);
            hin[2] = __builtin_fmaf(Ak.z, hin[2], Hk.z);
            hin[3] = __builtin_fmaf(Ak.w, hin[3], Hk.w);
          }
          // replay from the entering state
#pragma unroll
          for (int i = 0; i < TS; ++i) {
            const int row = seg * TS + i;
            const float cq = cur.cq[row][q];
#pragma unroll
            for (int j = 0; j < 4; ++j) hin[j] = __builtin_fmaf(av[i][j], hin[j], bv[i][j]);
            out.yq[g][row][ch] = dot_quad(cq, hin);
          }
          // the last segment's end state is the round's carry, and the
          // checkpoint of the chunk's next round (all 16 lanes of a group,
          // padded channels too: their state is their zero entering state)
          if (seg == SEG - 1) {
            fa.carry[r & 1][lane] = make_float4(hin[0], hin[1], hin[2], hin[3]);
            if (!rev && p.ckpt && r + 1 < rounds)
              *reinterpret_cast<float4*>(p.ckpt + ((b * p.ck_rounds + t0 / RT + r + 1) * p.ck_EDp + e) * 16 + 4 * g) =
                  make_float4(hin[0], hin[1], hin[2], hin[3]);
          }
        }
      }

      if (r + 1 < rounds) st.template commit<STAGE_SCAN>(p, nxt);
      __syncthreads();
    }
    st.template store_out<STAGE_SCAN>(p, rounds - 1, tile[(rounds - 1) & 1], out);
    if (SEG > 1 && wave == SEG - 1) {
      // the last round's carry (published before the round's closing barrier)
      const float4 c = fa.carry[(rounds - 1) & 1][lane];
      carry[0] = c.x, carry[1] = c.y, carry[2] = c.z, carry[3] = c.w;
    }

    if constexpr (!SPLIT) {
      float* h_out = rev ? p.g_first : p.h_last;
      if (h_out && wave == SEG - 1 && ch_ok)
        *reinterpret_cast<float4*>(h_out + (b * ED + e) * 16 + 4 * g) =
            make_float4(carry[0], carry[1], carry[2], carry[3]);
    } else if (rev) {
      gloc[0] = carry[0], gloc[1] = carry[1], gloc[2] = carry[2], gloc[3] = carry[3];
    }
    if (BIDIR) __syncthreads();
  }

  if constexpr (SPLIT && BIDIR) {
    // ---- publish the chunk's aggregates: sum of delta (float64), the
    // forward end state and the reverse start state, each from this chunk's
    // entering state (zero, or h0 / g0 at the sequence's ends) ----
    fa.sd[wave][lane] = sd_total;
    __syncthreads();
    if (wave == SEG - 1) {
      const int64_t slot = bg * p.nchunks + kchunk;
      if (g == 0) {
        double sum = 0.0;
#pragma unroll
        for (int s2 = 0; s2 < SEG; ++s2) sum += fa.sd[s2][lane];
        p.sdsum[slot * 16 + ch] = sum;
      }
      *reinterpret_cast<float4*>(p.state + slot * 256 + ch * 16 + 4 * g) =
          make_float4(carry[0], carry[1], carry[2], carry[3]);
      *reinterpret_cast<float4*>(p.gstate + slot * 256 + ch * 16 + 4 * g) =
          make_float4(gloc[0], gloc[1], gloc[2], gloc[3]);
    }
    return;
  }

  if constexpr (SPLIT && !BIDIR) {
    // ---- hand the chunk's end state to the next chunk -------------------
    // chunk aggregate: prod of a over the chunk = exp2(A log2e * sum delta),
    // the sum taken in float64 over all waves' segments
    fa.sd[wave][lane] = sd_total;
    __syncthreads();
    const int64_t slot = bg * p.nchunks + kchunk;
    float hin[4] = {0.f, 0.f, 0.f, 0.f};
    if (wave == SEG - 1) {
      double sum = 0.0;
#pragma unroll
      for (int s = 0; s < SEG; ++s) sum += fa.sd[s][lane];
      const float sdc = static_cast<float>(sum);
      float incl[4] = {carry[0], carry[1], carry[2], carry[3]};
      if (kchunk > 0) {
        int ok = 1;
        if (lane == 0) ok = wait_flag(p.flag + slot - 1, &p.hdr->err, p.spin_limit) ? 1 : 0;
        ok = __builtin_amdgcn_readfirstlane(ok);
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
        const float4 v = *reinterpret_cast<const float4*>(p.state + (slot - 1) * 256 + ch * 16 + 4 * g);
        hin[0] = v.x, hin[1] = v.y, hin[2] = v.z, hin[3] = v.w;
        if (!ok) hin[0] = hin[1] = hin[2] = hin[3] = __builtin_nanf("");  // a wait that gave up poisons the chunk
#pragma unroll
        for (int j = 0; j < 4; ++j) incl[j] = __builtin_fmaf(__builtin_amdgcn_exp2f(A2[j] * sdc), hin[j], carry[j]);
      }
      if (kchunk + 1 < p.nchunks) {
        *reinterpret_cast<float4*>(p.state + slot * 256 + ch * 16 + 4 * g) =
            make_float4(incl[0], incl[1], incl[2], incl[3]);
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "agent");
        if (lane == 0) __hip_atomic_store(p.flag + slot, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      } else if (p.h_last && ch_ok) {
        *reinterpret_cast<float4*>(p.h_last + (b * ED + e) * 16 + 4 * g) =
            make_float4(incl[0], incl[1], incl[2], incl[3]);
      }
      fa.carry[0][lane] = make_float4(hin[0], hin[1], hin[2], hin[3]);
    }
    if (kchunk == 0) return;  // uniform across the workgroup
    __syncthreads();
    {
      const float4 v = fa.carry[0][lane];
      hin[0] = v.x, hin[1] = v.y, hin[2] = v.z, hin[3] = v.w;
    }

    correct_pass<T, SEG, TS, VEC, GATE>(p, st, tile, out, b, t0, Lk, false, hin, A2, wave, ch, q, g);
  }
}

// Second kernel of the bidirectional split scan: one workgroup per (batch
// row, channel group, chunk) folds the chunks' aggregates into the states
// entering its chunk from either side, h_in = fold over the chunks before it
// (from h0) and g_in = fold over the chunks after it (from g0), writes h_last
// (last chunk) and g_first (first chunk), and corrects the chunk's outputs:
// the forward state's contribution from its first step on, the reverse
// state's from its last step backwards (in that order, so that a short chunk
// whose two corrections overlap adds both).
template <typename T, int SEG, int TS, bool VEC, bool GATE>
__global__ __launch_bounds__(64 * SEG) __attribute__((amdgpu_waves_per_eu(3))) void scan_bidir_join_kernel(
    const ScanArgs<T> p) {
  constexpr int RT = SEG * TS;
  constexpr int NT = 64 * SEG;
  constexpr int TPT = (8 * RT) / NT;
  __shared__ Tile<RT, GATE> tile[2];
  __shared__ OutTile<RT> out;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int q = lane & 15;
  const int g = q >> 2;
  const int ch = ((lane >> 4) << 2) | (q & 3);
  const int64_t L = p.L, ED = p.ED;
  const int64_t nbg = p.nblocks / p.nchunks;
  const int64_t kchunk = blockIdx.x / nbg, bg = blockIdx.x % nbg;
  const int64_t K = p.nchunks;
  const int64_t t0 = kchunk * p.chunk_len;
  const int64_t Lk = L - t0 < p.chunk_len ? L - t0 : p.chunk_len;
  const int64_t b = bg / p.ngroups;
  const int64_t e0 = (bg % p.ngroups) * 16;
  const int64_t e = e0 + ch;
  const bool ch_ok = e < ED;
  const int64_t ec = ch_ok ? e : ED - 1;
  float A2[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) A2[j] = p.A[ec * 16 + 4 * g + j] * kLog2e;

  // fold: state = prod(a over chunk j) * state + chunk j's own state
  auto fold = [&](float (&v)[4], const float* states, int64_t j) {
    const int64_t slot = bg * K + j;
    const float sdc = static_cast<float>(p.sdsum[slot * 16 + ch]);
    const float4 hj = *reinterpret_cast<const float4*>(states + slot * 256 + ch * 16 + 4 * g);
    const float hv[4] = {hj.x, hj.y, hj.z, hj.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) v[i] = __builtin_fmaf(__builtin_amdgcn_exp2f(A2[i] * sdc), v[i], hv[i]);
  };
  float hin[4] = {0.f, 0.f, 0.f, 0.f}, gin[4] = {0.f, 0.f, 0.f, 0.f};
  for (int64_t j = 0; j < kchunk; ++j) fold(hin, p.state, j);
  for (int64_t j = K - 1; j > kchunk; --j) fold(gin, p.gstate, j);
  if (wave == 0 && ch_ok) {
    if (kchunk == K - 1 && p.h_last) {
      float v[4] = {hin[0], hin[1], hin[2], hin[3]};
      fold(v, p.state, kchunk);
      *reinterpret_cast<float4*>(p.h_last + (b * ED + e) * 16 + 4 * g) = make_float4(v[0], v[1], v[2], v[3]);
    }
    if (kchunk == 0 && p.g_first) {
      float v[4] = {gin[0], gin[1], gin[2], gin[3]};
      fold(v, p.gstate, kchunk);
      *reinterpret_cast<float4*>(p.g_first + (b * ED + e) * 16 + 4 * g) = make_float4(v[0], v[1], v[2], v[3]);
    }
  }

  Stager<T, RT, TPT, false, VEC, GATE> st;
  st.init(p, tid, e0);
  if (kchunk > 0) correct_pass<T, SEG, TS, VEC, GATE>(p, st, tile, out, b, t0, Lk, false, hin, A2, wave, ch, q, g);
  // the forward correction's stores of y are read back by the reverse one
  __syncthreads();
  if (kchunk < K - 1) correct_pass<T, SEG, TS, VEC, GATE>(p, st, tile, out, b, t0, Lk, true, gin, A2, wave, ch, q, g);
}

// ---------------------------------------------------------------------------
// host-side validation
// ---------------------------------------------------------------------------
struct Sizes {
  int64_t seq;     // Bs * L * ED
  int64_t bc;      // Bs * L * N
  int64_t state;   // Bs * ED * N
  int64_t elem;    // bytes per x/delta/B/C/y element
};

// Bs, L and ED may be zero (empty tensors); N must be 16.
int check_sizes(int64_t Bs, int64_t L, int64_t ED, int64_t N, int dtype, Sizes* s) {
  if (Bs < 0 || L < 0 || ED < 0 || N <= 0) return SSM_ERR_DIM;
  int64_t t;
  if (!mul_nn(Bs, L, &t) || !mul_nn(t, ED, &s->seq) || !mul_nn(t, N, &s->bc)) return SSM_ERR_DIM;
  if (!mul_nn(Bs, ED, &t) || !mul_nn(t, N, &s->state)) return SSM_ERR_DIM;
  if (s->seq > INT64_MAX / 8 || s->state > INT64_MAX / 8) return SSM_ERR_DIM;
  if (dtype != SSM_F32 && dtype != SSM_BF16) return SSM_ERR_UNSUPPORTED;
  if (N != 16) return SSM_ERR_UNSUPPORTED;
  s->elem = dtype == SSM_F32 ? 4 : 2;
  return SSM_OK;
}

// Kernel configuration: SEG waves per workgroup, TS steps per wave per round.
constexpr int kSEG = 4, kTS = 8, kRT = kSEG * kTS;

// Workgroups of the split-sequence kernel that fit on one CU at once (the
// smallest over its instantiations), 0 if the runtime cannot tell.
int split_blocks_per_cu() {
  int best = 1 << 30;
  int n = 0;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, scan_chunked_kernel<float, kSEG, kTS, false, true, true, true>,
                                                   64 * kSEG, 0) != hipSuccess)
    return 0;
  best = std::min(best, n);
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, scan_chunked_kernel<float, kSEG, kTS, false, false, true, true>,
                                                   64 * kSEG, 0) != hipSuccess)
    return 0;
  best = std::min(best, n);
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, scan_chunked_kernel<uint16_t, kSEG, kTS, false, true, true, true>,
                                                   64 * kSEG, 0) != hipSuccess)
    return 0;
  best = std::min(best, n);
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, scan_chunked_kernel<uint16_t, kSEG, kTS, false, false, true, true>,
                                                   64 * kSEG, 0) != hipSuccess)
    return 0;
  return std::min(best, n);
}

// How a scan splits a sequence across workgroups: when there are fewer than
// two (batch row, 16-channel group) pairs per compute unit, cut the sequence
// into chunks (each at least 16 rounds long) so that about three workgroups
// per CU are in flight. The forward scan hands states from chunk to chunk
// inside the kernel (tickets make that safe whatever is resident); the
// bidirectional scan joins its chunks in a second kernel.
struct SplitPlan {
  int64_t nbg;        // (batch row, channel group) pairs
  int64_t nchunks;    // 1: no split
  int64_t chunk_len;
  // workspace layout. Forward: header, flags, states. Bidirectional: the
  // delta sums, the forward end states and the reverse start states.
  size_t flag_off, state_off, sd_off, gstate_off, bytes;
};

// Iterations of a hand-off wait before it gives up (s_sleep 4 each: about
// 7 s at 2^26). SSM_SPLIT_SPIN_LIMIT in the environment overrides it, so
// that a test can force the give-up path from the host.
unsigned split_spin_limit() {
  const char* e = std::getenv("SSM_SPLIT_SPIN_LIMIT");
  if (e && *e) {
    char* end = nullptr;
    const unsigned long v = std::strtoul(e, &end, 10);
    if (end && *end == '\0') return static_cast<unsigned>(std::min<unsigned long>(v, 1ul << 26));
  }
  return 1u << 26;
}

SplitPlan plan_split(int64_t Bs, int64_t L, int64_t ED, int bidir, int ncu) {
  SplitPlan sp{};
  sp.nbg = Bs * ((ED + 15) / 16);
  sp.nchunks = 1;
  sp.chunk_len = L;
  if (ncu > 0 && sp.nbg < 2 * static_cast<int64_t>(ncu)) {
    const int64_t per_cu = std::min<int64_t>(3, split_blocks_per_cu());  // workgroups resident per CU
    const int64_t want = per_cu * static_cast<int64_t>(ncu) / sp.nbg;
    const int64_t k = std::min<int64_t>(want, L / (16 * kRT));
    if (k >= 2) {
      const int64_t len = ((L + k - 1) / k + kRT - 1) / kRT * kRT;
      sp.chunk_len = len;
      sp.nchunks = (L + len - 1) / len;
    }
  }
  const size_t nslot = static_cast<size_t>(sp.nbg * sp.nchunks);
  if (sp.nchunks > 1 && bidir) {
    sp.sd_off = 0;
    sp.state_off = (nslot * 16 * 8 + 255) & ~static_cast<size_t>(255);
    sp.gstate_off = sp.state_off + nslot * 256 * 4;
    sp.bytes = sp.gstate_off + nslot * 256 * 4;
  } else if (sp.nchunks > 1) {
    sp.flag_off = sizeof(SplitHeader);
    sp.state_off = (sp.flag_off + static_cast<size_t>(sp.nbg * sp.nchunks) * 4 + 255) & ~static_cast<size_t>(255);
    sp.bytes = sp.state_off + static_cast<size_t>(sp.nbg * sp.nchunks) * 256 * 4;
  }
  return sp;
}

// the bidirectional bf16 scan keeps its reverse-time partial sums in float32
// at the start of the workspace; a split plan's buffers follow
size_t partial_bytes(int64_t seq, int dtype, int bidir) {
  return (bidir && dtype == SSM_BF16) ? (static_cast<size_t>(seq) * 4 + 255) & ~static_cast<size_t>(255) : 0;
}

size_t workspace_bytes(int64_t Bs, int64_t L, int64_t ED, int64_t N, int dtype, int bidir) {
  Sizes s;
  if (check_sizes(Bs, L, ED, N, dtype, &s) != SSM_OK || s.seq == 0) return 0;
  return partial_bytes(s.seq, dtype, bidir) + plan_split(Bs, L, ED, bidir, device_cus()).bytes;
}

// Bytes of the round checkpoints (Bs, ceil(L / kRT), 16 ceil(ED / 16), 16)
// float32, or 0 when the sizes overflow
size_t ckpt_bytes(int64_t Bs, int64_t L, int64_t ED) {
  if (Bs < 0 || L < 0 || ED < 0) return 0;
  int64_t t;
  const int64_t rounds = (L + 31) / 32, EDp = (ED + 15) / 16 * 16;
  if (!mul_nn(Bs, rounds, &t) || !mul_nn(t, EDp, &t) || !mul_nn(t, 16, &t) || t > INT64_MAX / 4) return 0;
  return static_cast<size_t>(t) * 4;
}

int validate(const void* x, const void* delta, const float* A, const void* B, const void* C, const float* D,
             const float* h0, const float* g0, const ssm_scan_options* opts, const void* y, const float* h_last, const float* g_first, int64_t Bs, int64_t L, int64_t ED,
             int64_t N, int dtype, const void* ws, size_t ws_bytes, int bidir, Sizes* s, bool want_ck = false,
             const void* ckpt = nullptr, size_t ck_bytes = 0) {
  int rc = check_sizes(Bs, L, ED, N, dtype, s);
  if (rc != SSM_OK) return rc;
  const size_t ck_need = want_ck && s->seq > 0 ? ckpt_bytes(Bs, L, ED) : 0;
  if (want_ck && s->seq > 0) {
    if (ck_need == 0) return SSM_ERR_DIM;
    if (!ckpt) return SSM_ERR_NULL;
    if (!aligned16(ckpt)) return SSM_ERR_UNSUPPORTED;
    if (ck_bytes < ck_need) return SSM_ERR_WORKSPACE;
  }
  // a buffer with no elements may be NULL
  if ((s->seq > 0 && (!x || !delta || !y)) || (s->bc > 0 && (!B || !C)) || (ED > 0 && !A)) return SSM_ERR_NULL;
  const float* dt_bias = opts ? opts->dt_bias : nullptr;
  const void* z = opts ? opts->z : nullptr;
  if (opts && !(opts->dt_min <= opts->dt_max)) return SSM_ERR_ARG;  // also catches NaN
  const void* ptrs[] = {x, delta, A, B, C, D, h0, g0, dt_bias, z, y, h_last, g_first, ws};
  for (const void* p : ptrs)
    if (p && !aligned16(p)) return SSM_ERR_UNSUPPORTED;
  size_t need = workspace_bytes(Bs, L, ED, N, dtype, bidir);
  if (need > 0 && (!ws || ws_bytes < need)) return SSM_ERR_WORKSPACE;

  Range in[] = {rng(x, s->seq * s->elem), rng(delta, s->seq * s->elem), rng(A, ED * N * 4),
                rng(B, s->bc * s->elem), rng(C, s->bc * s->elem), rng(D, D ? ED * 4 : 0),
                rng(h0, h0 ? s->state * 4 : 0), rng(g0, g0 ? s->state * 4 : 0), rng(dt_bias, dt_bias ? ED * 4 : 0),
                rng(z, z ? s->seq * s->elem : 0)};
  Range out[5];
  int nout = 0;
  out[nout++] = rng(y, s->seq * s->elem);
  if (h_last) out[nout++] = rng(h_last, s->state * 4);
  if (g_first) out[nout++] = rng(g_first, s->state * 4);
  if (need > 0) out[nout++] = rng(ws, static_cast<int64_t>(need));
  if (ck_need > 0) out[nout++] = rng(ckpt, static_cast<int64_t>(ck_need));
  for (int i = 0; i < nout; ++i) {
    if (out[i].hi == out[i].lo) continue;
    for (const Range& r : in)
      if (r.hi > r.lo && overlap(out[i], r)) return SSM_ERR_ALIAS;
    for (int j = i + 1; j < nout; ++j)
      if (out[j].hi > out[j].lo && overlap(out[i], out[j])) return SSM_ERR_ALIAS;
  }
  return SSM_OK;
}

// LDS of one workgroup of the forward kernel
template <bool GATE, bool SPLIT>
constexpr size_t scan_lds_bytes() {
  return sizeof(Tile<kRT, GATE>) * 2 + sizeof(OutTile<kRT>) + sizeof(FoldArea<kSEG, SPLIT>) + 16;
}

// A launch with more workgroups than 3 per compute unit (which is what the
// gated, bidirectional and split kernels hold) runs the plain kernel built
// for 4 per compute unit (at most 128 VGPRs, under 40 KB of LDS): the last
// workgroups then start sooner (bf16 4x8192x5120: 861 -> 813 us).
template <typename T, bool BIDIR, bool VEC, bool SPLIT>
void launch_one(const ScanArgs<T>& a, int64_t nblk, hipStream_t stream) {
  const dim3 grid(static_cast<unsigned>(nblk)), block(64 * kSEG);
  const int ncu = device_cus();
  if constexpr (!BIDIR && !SPLIT) {
    if (!a.z && ncu > 0 && nblk > 3 * static_cast<int64_t>(ncu)) {
      const size_t dyn = spread_lds(nblk, scan_lds_bytes<false, false>(), 4);
      hipLaunchKernelGGL((scan_chunked_kernel<T, kSEG, kTS, false, VEC, false, false, 4>), grid, block, dyn, stream, a);
      return;
    }
  }
  const size_t dyn = spread_lds(nblk, scan_lds_bytes<true, SPLIT>(), 3);
  if (a.z)
    hipLaunchKernelGGL((scan_chunked_kernel<T, kSEG, kTS, BIDIR, VEC, SPLIT, true>), grid, block, dyn, stream, a);
  else
    hipLaunchKernelGGL((scan_chunked_kernel<T, kSEG, kTS, BIDIR, VEC, SPLIT, false>), grid, block, dyn, stream, a);
}

template <typename T>
int launch_scan(const void* x, const void* delta, const float* A, const void* B, const void* C, const float* D,
                const float* h0, const float* g0, const ssm_scan_options* opts, void* y, float* h_last, float* g_first, int64_t Bs, int64_t L, int64_t ED, int bidir, void* ws,
                hipStream_t stream, float* ckpt = nullptr) {
  const int64_t ngroups = (ED + 15) / 16;
  const SplitPlan sp = plan_split(Bs, L, ED, bidir, device_cus());
  const int64_t nblk = sp.nbg * sp.nchunks;
  if (nblk > INT32_MAX / 2) return SSM_ERR_DIM;
  ScanArgs<T> a;
  a.x = static_cast<const T*>(x);
  a.dl = static_cast<const T*>(delta);
  a.A = A;
  a.B = static_cast<const T*>(B);
  a.C = static_cast<const T*>(C);
  a.D = D;
  a.h0 = h0;
  a.g0 = bidir ? g0 : nullptr;
  a.dt_bias = opts ? opts->dt_bias : nullptr;
  a.dt_softplus = opts && opts->dt_softplus ? 1 : 0;
  a.dt_min = opts ? opts->dt_min : -INFINITY;
  a.dt_max = opts ? opts->dt_max : INFINITY;
  a.dt_pre = (a.dt_bias || a.dt_softplus || a.dt_min > -INFINITY || a.dt_max < INFINITY) ? 1 : 0;
  a.z = opts ? static_cast<const T*>(opts->z) : nullptr;
  a.y = static_cast<T*>(y);
  a.part = bidir ? (std::is_same<T, float>::value ? reinterpret_cast<float*>(y) : static_cast<float*>(ws)) : nullptr;
  a.h_last = h_last;
  a.g_first = bidir ? g_first : nullptr;
  a.L = L;
  a.ED = ED;
  a.ngroups = static_cast<int>(ngroups);
  a.nblocks = static_cast<int>(nblk);
  a.remap = (nblk % 8 == 0) ? 1 : 0;
  a.rot_ncu = rotation_cus(nblk);
  a.nchunks = static_cast<int>(sp.nchunks);
  a.chunk_len = sp.chunk_len;
  a.spin_limit = split_spin_limit();
  a.hdr = nullptr;
  a.flag = nullptr;
  a.state = nullptr;
  a.sdsum = nullptr;
  a.gstate = nullptr;
  a.ckpt = ckpt;  // the forward direction's round states (both scans)
  a.ck_rounds = (L + kRT - 1) / kRT;
  a.ck_EDp = ngroups * 16;
  const bool split = sp.nchunks > 1;
  if (split && bidir) {
    char* w = static_cast<char*>(ws) + partial_bytes(Bs * L * ED, std::is_same<T, float>::value ? SSM_F32 : SSM_BF16, 1);
    a.sdsum = reinterpret_cast<double*>(w + sp.sd_off);
    a.state = reinterpret_cast<float*>(w + sp.state_off);
    a.gstate = reinterpret_cast<float*>(w + sp.gstate_off);
  } else if (split) {
    char* w = static_cast<char*>(ws);
    a.hdr = reinterpret_cast<SplitHeader*>(w);
    a.flag = reinterpret_cast<int*>(w + sp.flag_off);
    a.state = reinterpret_cast<float*>(w + sp.state_off);
    const int64_t words = static_cast<int64_t>(sp.state_off / 4);
    hipLaunchKernelGGL(zero_words_kernel, dim3(static_cast<unsigned>(std::min<int64_t>((words + 255) / 256, 1024))),
                       dim3(256), 0, stream, reinterpret_cast<unsigned*>(w), words);
  }
  const bool vec = (ED % 4) == 0;
  if (bidir && split) {
    // both directions of every chunk from its own entering states, then the
    // join: entering states from the chunks' aggregates, and corrections
    if (vec) launch_one<T, true, true, true>(a, nblk, stream);
    else launch_one<T, true, false, true>(a, nblk, stream);
    const dim3 grid(static_cast<unsigned>(nblk)), block(64 * kSEG);
    if (a.z) {
      if (vec) hipLaunchKernelGGL((scan_bidir_join_kernel<T, kSEG, kTS, true, true>), grid, block, 0, stream, a);
      else hipLaunchKernelGGL((scan_bidir_join_kernel<T, kSEG, kTS, false, true>), grid, block, 0, stream, a);
    } else {
      if (vec) hipLaunchKernelGGL((scan_bidir_join_kernel<T, kSEG, kTS, true, false>), grid, block, 0, stream, a);
      else hipLaunchKernelGGL((scan_bidir_join_kernel<T, kSEG, kTS, false, false>), grid, block, 0, stream, a);
    }
  } else if (bidir) {
    if (vec) launch_one<T, true, true, false>(a, nblk, stream);
    else launch_one<T, true, false, false>(a, nblk, stream);
  } else if (split) {
    if (vec) launch_one<T, false, true, true>(a, nblk, stream);
    else launch_one<T, false, false, true>(a, nblk, stream);
  } else {
    if (vec) launch_one<T, false, true, false>(a, nblk, stream);
    else launch_one<T, false, false, false>(a, nblk, stream);
  }
  return hipGetLastError() == hipSuccess ? SSM_OK : SSM_ERR_LAUNCH;
}

int run(const void* x, const void* delta, const float* A, const void* B, const void* C, const float* D,
        const float* h0, const float* g0, const ssm_scan_options* opts, void* y,
        float* h_last, float* g_first, int64_t Bs, int64_t L, int64_t ED, int64_t N, int dtype, void* ws,
        size_t ws_bytes, void* stream, int bidir, bool want_ck = false, float* ckpt = nullptr, size_t ck_bytes = 0) {
  Sizes s;
  if (!bidir) g0 = nullptr;
  int rc = validate(x, delta, A, B, C, D, h0, g0, opts, y, h_last, g_first, Bs, L, ED, N, dtype, ws, ws_bytes, bidir, &s,
                    want_ck, ckpt, ck_bytes);
  if (rc != SSM_OK) return rc;
  hipStream_t st = static_cast<hipStream_t>(stream);
  if (s.seq == 0) {
    // nothing to scan. Over an empty sequence each state stays where it
    // entered (h_last = h0, g_first = g0, or zero).
    const bool ok = fill_async(h_last, h0, s.state * 4, st) && fill_async(bidir ? g_first : nullptr, g0,
                                                                          s.state * 4, st);
    return ok ? SSM_OK : SSM_ERR_LAUNCH;
  }
  float* ck = want_ck ? ckpt : nullptr;
  if (dtype == SSM_F32)
    return launch_scan<float>(x, delta, A, B, C, D, h0, g0, opts, y, h_last, g_first, Bs, L, ED, bidir, ws, st, ck);
  return launch_scan<uint16_t>(x, delta, A, B, C, D, h0, g0, opts, y, h_last, g_first, Bs, L, ED, bidir, ws, st, ck);
}

}  // namespace

// ---------------------------------------------------------------------------
// The split-sequence hand-off buffer of ssm_scan_fwd_noalloc: a file-scope
// device array, one copy per device, held until the process ends. A split
// plan needs a 256-byte header, one flag word and one 16 x 16 float32 state
// per chunk (at most three chunks per compute unit): 1 MiB covers every plan
// on a device of up to 340 compute units.
// ---------------------------------------------------------------------------
static __device__ __align__(256) unsigned char scratch[SSM_NOALLOC_SCRATCH_BYTES];

namespace {

constexpr int kMaxDevices = 64;
std::atomic<void*> g_scratch_ptr[kMaxDevices];  // device address of `scratch` per device, once resolved
std::mutex g_scratch_mu;

// The device address of `scratch` on the current device, resolved once per
// device with that device current. (In host code the name `scratch` is a
// host-side stand-in, not a device address: only this pointer may reach a
// kernel or a copy.)
int scratch_on_current_device(void** out) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return SSM_ERR_LAUNCH;
  if (dev < 0 || dev >= kMaxDevices) return SSM_ERR_UNSUPPORTED;
  void* p = g_scratch_ptr[dev].load(std::memory_order_acquire);
  if (!p) {
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    p = g_scratch_ptr[dev].load(std::memory_order_relaxed);
    if (!p) {
      if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return SSM_ERR_LAUNCH;
      g_scratch_ptr[dev].store(p, std::memory_order_release);
    }
  }
  *out = p;
  return SSM_OK;
}

}  // namespace

extern "C" {

size_t ssm_scan_workspace_bytes(int64_t Bs, int64_t L, int64_t ED, int64_t N, int dtype, int bidir) {
  return workspace_bytes(Bs, L, ED, N, dtype, bidir);
}

int ssm_scan_fwd(const void* x, const void* delta, const float* A, const void* B, const void* C, const float* D,
                 const float* h0, const ssm_scan_options* opts, void* y, float* h_last, int64_t Bs, int64_t L,
                 int64_t ED, int64_t N, int dtype, void* workspace, size_t workspace_bytes, void* stream) {
  return run(x, delta, A, B, C, D, h0, nullptr, opts, y, h_last, nullptr, Bs, L, ED, N, dtype, workspace,
             workspace_bytes, stream, 0);
}

size_t ssm_scan_ckpt_bytes(int64_t Bs, int64_t L, int64_t ED, int64_t N) {
  if (N != 16) return 0;
  return ckpt_bytes(Bs, L, ED);
}

int ssm_scan_fwd_ckpt(const void* x, const void* delta, const float* A, const void* B, const void* C, const float* D,
                      const float* h0, const ssm_scan_options* opts, void* y, float* h_last, float* ckpt,
                      size_t ckpt_bytes, int64_t Bs, int64_t L, int64_t ED, int64_t N, int dtype, void* workspace,
                      size_t workspace_bytes, void* stream) {
  return run(x, delta, A, B, C, D, h0, nullptr, opts, y, h_last, nullptr, Bs, L, ED, N, dtype, workspace,
             workspace_bytes, stream, 0, true, ckpt, ckpt_bytes);
}

int ssm_scan_bidir_fwd(const void* x, const void* delta, const float* A, const void* B, const void* C,
                       const float* D, const float* h0, const float* g0, const ssm_scan_options* opts, void* y,
                       float* h_last, float* g_first, int64_t Bs, int64_t L, int64_t ED, int64_t N, int dtype,
                       void* workspace, size_t workspace_bytes, void* stream) {
  return run(x, delta, A, B, C, D, h0, g0, opts, y, h_last, g_first, Bs, L, ED, N, dtype, workspace, workspace_bytes,
             stream, 1);
}

int ssm_scan_bidir_fwd_ckpt(const void* x, const void* delta, const float* A, const void* B, const void* C,
                            const float* D, const float* h0, const float* g0, const ssm_scan_options* opts, void* y,
                            float* h_last, float* g_first, float* ckpt, size_t ckpt_bytes, int64_t Bs, int64_t L,
                            int64_t ED, int64_t N, int dtype, void* workspace, size_t workspace_bytes, void* stream) {
  return run(x, delta, A, B, C, D, h0, g0, opts, y, h_last, g_first, Bs, L, ED, N, dtype, workspace, workspace_bytes,
             stream, 1, true, ckpt, ckpt_bytes);
}

int ssm_scan_fwd_noalloc(const void* x, const void* delta, const float* A, const void* B, const void* C,
                         const float* D, const float* h0, const ssm_scan_options* opts, void* y, float* h_last,
                         int64_t Bs, int64_t L, int64_t ED, int64_t N, int dtype, void* stream) {
  Sizes s;
  const int rc = check_sizes(Bs, L, ED, N, dtype, &s);
  if (rc != SSM_OK) return rc;
  const size_t need = s.seq == 0 ? 0 : workspace_bytes(Bs, L, ED, N, dtype, 0);
  if (need > SSM_NOALLOC_SCRATCH_BYTES) return SSM_ERR_WORKSPACE;
  void* ws = nullptr;
  if (need > 0) {
    const int r2 = scratch_on_current_device(&ws);
    if (r2 != SSM_OK) return r2;
  }
  return run(x, delta, A, B, C, D, h0, nullptr, opts, y, h_last, nullptr, Bs, L, ED, N, dtype, ws, need, stream, 0);
}

int ssm_scan_fwd_status(const void* workspace, size_t workspace_bytes, int64_t Bs, int64_t L, int64_t ED,
                        int64_t N, int dtype, void* stream) {
  Sizes s;
  int rc = check_sizes(Bs, L, ED, N, dtype, &s);
  if (rc != SSM_OK) return rc;
  hipStream_t st = static_cast<hipStream_t>(stream);
  if (hipStreamSynchronize(st) != hipSuccess) return SSM_ERR_LAUNCH;
  if (s.seq == 0) return SSM_OK;
  const SplitPlan sp = plan_split(Bs, L, ED, 0, device_cus());
  if (sp.nchunks <= 1) return SSM_OK;  // no hand-off in this call
  if (!workspace) {
    // the internal buffer of ssm_scan_fwd_noalloc on the current device
    void* p = nullptr;
    const int r2 = scratch_on_current_device(&p);
    if (r2 != SSM_OK) return r2;
    workspace = p;
    workspace_bytes = SSM_NOALLOC_SCRATCH_BYTES;
  }
  if (workspace_bytes < sp.bytes) return SSM_ERR_WORKSPACE;
  unsigned err = 0;
  if (hipMemcpy(&err, workspace, sizeof(err), hipMemcpyDeviceToHost) != hipSuccess) return SSM_ERR_LAUNCH;
  return err ? SSM_ERR_HANDOFF : SSM_OK;
}

const char* ssm_status_str(int status) {
  switch (status) {
    case SSM_OK: return "ok";
    case SSM_ERR_NULL: return "a required pointer is NULL";
    case SSM_ERR_DIM: return "a dimension is negative (or not positive where it must be) or the sizes overflow";
    case SSM_ERR_UNSUPPORTED: return "unsupported N or dtype, or a pointer not aligned to 16 bytes";
    case SSM_ERR_ALIAS: return "an output overlaps an input, another output or the workspace";
    case SSM_ERR_WORKSPACE: return "workspace missing or smaller than ssm_scan_workspace_bytes()";
    case SSM_ERR_LAUNCH: return "the HIP runtime rejected a kernel launch";
    case SSM_ERR_ARG: return "an option is invalid (dt_min > dt_max, or a NaN bound)";
    case SSM_ERR_HANDOFF: return "a split-sequence hand-off wait gave up; the affected outputs are NaN";
    default: return "unknown status";
  }
}

}  // extern "C"
