// Speculative-sampling verification step for MI355X (CDNA4, gfx950): HIP kernels + C ABI.
//
// The step (pages cited in include/spec_verify.h by title and section): per request, accept
// draft x_i with probability min(1, p_i(x_i)/q_i(x_i)), stop at the first rejection j,
// and emit a draw from max(p_j - q_j, 0) there, or from p_gamma when nothing was rejected;
// at temperature zero, compare each draft with the target argmax instead.
//
// A verification call is two launches on the caller's stream, neither waiting for the host,
// or one launch for small calls (below):
//
//  k_rowstats  The HBM-bound stream.  Every needed logit row is read exactly once, cut into
//              16K-element tiles, one workgroup per (row slot, slice) on a 2-D grid; slots a
//              request does not use exit at once.  The workgroup loads its tile with 16-byte
//              nontemporal loads straight into registers, takes the tile maximum (packed
//              16-bit integer compares for bf16, wave shuffles, one LDS exchange), then sums
//              2^((z - M) c), c = log2(e)/T: fp32 terms in a fixed pairwise tree over each
//              thread's 64 elements, fp64 beyond.  Greedy rows (T = 0) reduce to (max, lowest
//              argmax).  Output: one partial per (row, slice), and per row slot a record of
//              the row's logit at its draft token, the token and its accept uniform.
//
//  k_finish    Workgroups (slice of the vocabulary, request).  Each one (1) merges its
//              request's row partials (a group of lanes per row slot, one lane per tile,
//              fp64) and (2) runs the accept tests lane-parallel (p(x), q(x) in fp64 from the
//              captured logits) with the first rejection from ballot + find-first-set; slice 0
//              writes the outputs.  For a sampled request every slice then (3) streams its part
//              of the stop row(s) into one fp64 sum of S_t (p_k - q_k)_+ (or S_t p_k for the
//              bonus) per 64-unit chunk, and the last slice to finish (4) draws: a block scan
//              over the request's chunk sums picks the chunk holding u * R, a wavefront scan
//              over its 64 units picks the unit, and a walk over the unit's elements gives the
//              token.  The chunk sums cross workgroups as device-scope atomic stores and loads,
//              ordered by a per-request arrival counter (which k_rowstats clears), so no cache
//              writeback is needed inside the kernel.
//
// One launch for small calls, where it measured faster, or when the probe's path field asks:
//
//  k_greedy1   Greedy calls: k_rowstats' tiles over the target rows; the last tile of a
//              request to finish merges the request's partials and writes its outputs.
//
//  k_onepass   Sampling calls whose workgroups fit on the device at once: k_rowstats' tiles
//              over every row; the request's tiles meet on an arrival counter, sum one span of
//              the stop row(s) each, and the one completing the last span draws, as k_finish
//              does.  Waits are bounded and a workgroup that stops waiting hands its span to
//              the last arrival, so no wait can change a result.
//
// Per-request counters sit one per 128-byte line: atomics on one line serialise.
//
// After a call, for a serving loop that stays on the device: k_commit appends each
// request's emitted tokens to its history and counts the step; k_ngram (+ k_ngram_pack)
// drafts the next step by prompt lookup.
//
// Numerics: logits convert exactly to fp32; exponent arguments carry the temperature as a
// two-float constant, so rounding never shifts the temperature, and their shifts are kept
// exact in fp64 when partials are combined; every sum beyond one thread's terms is fp64.
// Merged row sums are the normaliser sum_k exp((z_k - max)/T).
#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>

#include <atomic>
#include <cmath>
#include <cstddef>
#include <cstdint>
#include <type_traits>

#include "spec_verify.h"

namespace {

constexpr int kThreads = 256;                // 4 wavefronts of 64
constexpr int kWaves = kThreads / 64;
constexpr int64_t kTileElems = 16384;        // k_rowstats tile
constexpr int kRsThreads = 256;              // k_rowstats workgroup: 64 elements per thread
constexpr int kRsWaves = kRsThreads / 64;
constexpr int kMaxSlices = 64;               // finest cut of rows in small problems
constexpr int kSmallGrid = 1024;             // below this many tiles, cut rows finer
constexpr int64_t kMaxGridY = 65535;         // k_rowstats slots per grid row (y), z covers more
constexpr int kFinRU = 4;                    // k_finish: units per thread per row in flight
constexpr int kFinPassUnits = kThreads * kFinRU;  // k_finish: stop-row units per pass
constexpr int kFinGrid = 1024;               // k_finish workgroups aimed for
constexpr int kChunkUnits = 64;              // residual sums: one per 64 units (a wavefront load)
constexpr int kOneMaxB = 2048;               // requests the one-launch counters cover
constexpr int kCounterStride = 32;           // one counter per 128-byte line: atomics on a line
                                             // serialise, so requests must not share one
constexpr uint32_t kSpinLimit = 1u << 12;    // default polls before a one-launch workgroup
                                             // stops waiting (a poll is a device-scope round
                                             // trip, ~1 us: milliseconds, where a request's
                                             // tiles arrive within microseconds)
constexpr int64_t kMaxV = int64_t(1) << 24;
constexpr double kLog2e = 1.4426950408889634074;
constexpr size_t kAlign = 256;

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));


// Per (row, V-slice) result of k_rowstats.  Sampled rows: m = raw max of the slice,
// s = sum of 2^((z - m) c).  Greedy rows: m = raw max, idx = lowest index attaining it.
struct alignas(16) Partial {
  float m;
  int32_t idx;
  double s;
};

enum : int32_t { kModeNone = 0, kModeResidual = 1, kModeBonus = 2 };

// Per row slot, from k_rowstats for k_finish's accept tests: the row's logit at its draft
// token (sampled rows), and for target rows 0..gamma_b-1 the draft token and its accept
// uniform, so k_finish reads all of them in its first round trip.
struct alignas(16) SlotRec {
  float z;
  int32_t tok;
  float u;
  int32_t pad;
};

// What the residual weights and the draw of a sampled request's stop row j need.
struct alignas(16) Stop {
  int32_t mode;
  float mt, md;              // maxima of target / draft row j
  float c_hi, c_lo;          // log2(e)/T as a two-float constant
  float rho_hi, rho_lo;      // S_t / S_d as a two-float constant
  double st;                 // S_t
  int64_t trow;              // target row j: also the output slot of the emitted token
  int64_t drow;              // draft row j (read in residual mode only)
};

struct Params {
  const void *target, *draft;
  const int32_t *tokens;
  const float *uniforms, *temps;
  const int32_t *cu;
  int32_t B, gamma;
  int64_t V;
  int32_t *out_tokens, *out_n;
  Partial *parts;
  SlotRec *rec;             // [B][spr] per row slot: logit at the draft token, token, uniform
  double *chunk_sums;       // [B][chunk_stride] residual sums per 64-unit chunk
  int64_t chunk_stride;
  uint32_t *done;           // k_finish slices of request b finished, at [b * kCounterStride]
                            // (k_rowstats clears it)
  uint32_t *arrive, *odone; // one-launch counters, request b's at [b * kCounterStride]
                            // (arrive: a 64-bit word, arrivals and spans handed over; odone:
                            // completed spans): zero before and after every call
  int32_t nslice;           // k_finish workgroups per request
  int64_t slice_units;      // stop-row units per k_finish workgroup (a multiple of 64)
  int32_t spr;              // row slots per request: 2*gamma+1 (sample) or gamma+1 (greedy)
  int32_t nsplit;           // k_rowstats tiles (slices) per row
  int64_t split_len;        // elements per slice: one tile, or less for small problems
  int32_t greedy_all;
  uint32_t spin_limit;      // polls before a one-launch workgroup stops waiting
  double *p_x, *q_x, *row_sum_t, *row_sum_d, *resid_mass;
  float *row_max_t, *row_max_d;
};

// ------------------------------------------------------------------ small helpers

__device__ __forceinline__ int64_t ceil_div_dev(int64_t a, int64_t b) { return (a + b - 1) / b; }

__device__ __forceinline__ void request(const Params &P, int32_t b, int64_t &dbase,
                                        int32_t &gb, float &T) {
  if (P.cu) {
    const int32_t lo = P.cu[b], hi = P.cu[b + 1];
    dbase = lo;
    gb = hi - lo;
  } else {
    dbase = (int64_t)b * P.gamma;
    gb = P.gamma;
  }
  gb = gb < 0 ? 0 : (gb > P.gamma ? P.gamma : gb);  // memory safety on a malformed CSR
  T = P.greedy_all ? 0.f : P.temps[b];
}

struct TempConst {
  double c;  // c_hi + c_lo exactly: log2(e)/T to ~1e-16
  float c_hi, c_lo;
};

// c = log2(e)/T as c_hi + c_lo with c_lo > 0 strictly (c_hi is c rounded down, one ulp lower
// where c is a float): a masked logit z = -inf then gives z c_hi + z c_lo = -inf and a term of
// exactly 0, never -inf + inf or -inf * 0.  c is kept in [2^-80, 1e38]: temperatures below
// ~1.4e-38 act as ~1.4e-38, and above ~1.7e24 (T = +inf included) as ~1.7e24, where every
// finite logit's term is 1 and the distribution is uniform over the unmasked tokens; at the
// lower bound c_lo (~c 2^-24) is still a normal float.
constexpr double kMinTempConst = 8.271806125530277e-25;  // 2^-80
__device__ __forceinline__ TempConst temp_const(float T) {
  double c = kLog2e / (double)T;
  if (c > 1e38) c = 1e38;
  if (!(c >= kMinTempConst)) c = kMinTempConst;
  float hi = (float)c;
  if ((double)hi >= c) hi = __uint_as_float(__float_as_uint(hi) - 1u);  // hi > 0: one ulp down
  const float lo = (float)(c - (double)hi);
  return {(double)hi + (double)lo, hi, lo};
}

template <int DT>
__device__ __forceinline__ float logit_at(const void *base, int64_t idx) {
  if constexpr (DT == SPEC_F32) {
    return static_cast<const float *>(base)[idx];
  } else {
    const uint32_t h = static_cast<const uint16_t *>(base)[idx];
    return __uint_as_float(h << 16);
  }
}

template <int DT>
__device__ __forceinline__ const void *row_ptr(const void *base, int64_t row, int64_t V) {
  constexpr int64_t es = DT == SPEC_F32 ? 4 : 2;
  return static_cast<const char *>(base) + row * V * es;
}

// Load units.  VEC: rows are 16-byte aligned and a unit is one 16-byte load (4 fp32 or
// 8 bf16); otherwise a unit is one element.
template <int DT, bool VEC>
struct Unit {
  static constexpr int W = VEC ? (DT == SPEC_F32 ? 4 : 8) : 1;
  using Raw = typename std::conditional<VEC, u32x4, float>::type;   // one unit in registers
  using Store = typename std::conditional<                            // one unit in memory
      VEC, u32x4, typename std::conditional<DT == SPEC_F32, float, uint16_t>::type>::type;

  template <bool NT>
  __device__ static __forceinline__ Raw load(const Store *base, int64_t u) {
    if constexpr (VEC) {
      if constexpr (NT) return __builtin_nontemporal_load(base + u);
      else return base[u];
    } else if constexpr (DT == SPEC_F32) {
      return base[u];
    } else {
      return __uint_as_float((uint32_t)base[u] << 16);
    }
  }
  // Filler for units past the row end: the most negative finite value (its term is 0).
  __device__ static __forceinline__ Raw filler() {
    if constexpr (VEC) {
      const uint32_t v = DT == SPEC_F32 ? 0xff7fffffu : 0xff7fff7fu;
      return u32x4{v, v, v, v};
    } else {
      return DT == SPEC_F32 ? -3.40282347e38f : __uint_as_float(0xff7f0000u);
    }
  }
  // Exact maximum over a thread's units.  bf16 pairs are compared as packed 16-bit integers,
  // one instruction per pair and no conversion: read as int16, bf16 patterns order every
  // non-negative value correctly and place every negative value below them; among patterns
  // with the sign bit set, the smallest unsigned pattern is the largest value.  So a
  // non-negative signed maximum is the maximum, and otherwise (all values negative) the
  // unsigned minimum is.
  template <int N>
  __device__ static __forceinline__ float thread_max(const Raw (&r)[N]) {
    if constexpr (VEC && DT == SPEC_BF16) {
      typedef int16_t i16x2 __attribute__((ext_vector_type(2)));
      typedef uint16_t u16x2 __attribute__((ext_vector_type(2)));
      i16x2 mi = {INT16_MIN, INT16_MIN};
      u16x2 mu = {UINT16_MAX, UINT16_MAX};
#pragma unroll
      for (int j = 0; j < N; ++j) {
        const uint32_t w[4] = {r[j].x, r[j].y, r[j].z, r[j].w};
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          mi = __builtin_elementwise_max(mi, __builtin_bit_cast(i16x2, w[q]));
          mu = __builtin_elementwise_min(mu, __builtin_bit_cast(u16x2, w[q]));
        }
      }
      const int16_t smax = mi.x > mi.y ? mi.x : mi.y;
      const uint16_t umin = mu.x < mu.y ? mu.x : mu.y;
      const uint32_t pat = smax >= 0 ? (uint32_t)(uint16_t)smax : (uint32_t)umin;
      return __uint_as_float(pat << 16);
    } else {
      float m = -INFINITY;
#pragma unroll
      for (int j = 0; j < N; ++j) {
        if constexpr (!VEC) {
          m = fmaxf(m, r[j]);
        } else {
          m = fmaxf(fmaxf(m, __uint_as_float(r[j].x)),
                    fmaxf(fmaxf(__uint_as_float(r[j].y), __uint_as_float(r[j].z)),
                          __uint_as_float(r[j].w)));
        }
      }
      return m;
    }
  }
  __device__ static __forceinline__ void cvt(const Raw &r, float (&x)[W]) {
    if constexpr (!VEC) {
      x[0] = r;
    } else if constexpr (DT == SPEC_F32) {
      x[0] = __uint_as_float(r.x);
      x[1] = __uint_as_float(r.y);
      x[2] = __uint_as_float(r.z);
      x[3] = __uint_as_float(r.w);
    } else {
      x[0] = __uint_as_float(r.x << 16);
      x[1] = __uint_as_float(r.x & 0xffff0000u);
      x[2] = __uint_as_float(r.y << 16);
      x[3] = __uint_as_float(r.y & 0xffff0000u);
      x[4] = __uint_as_float(r.z << 16);
      x[5] = __uint_as_float(r.z & 0xffff0000u);
      x[6] = __uint_as_float(r.w << 16);
      x[7] = __uint_as_float(r.w & 0xffff0000u);
    }
  }
};

// Exponent arguments of the terms 2^(z c - shift):
//  shifted: shift = m c exactly, computed as (z - m) c_hi + (z - m) c_lo with the exact
//           difference first; safe for any m and c.
//  folded:  shift = K = fp32(m c), computed as (z c_hi - K) + z c_lo: two FMAs.  The inner
//           FMA rounds only the small difference, and z c_lo is added to it last, so no part
//           of c is lost.  Used when |m| c < 2^22: then |m c - K| < 1/2, no term overflows.
// Sums in either form are brought to the shifted form (shift m c) exactly in fp64.
__device__ __forceinline__ float arg_shifted(float z, float m, float c_hi, float c_lo) {
  const float d = z - m;
  return fmaf(d, c_hi, d * c_lo);
}
__device__ __forceinline__ float arg_folded(float z, float K, float c_hi, float c_lo) {
  return fmaf(z, c_lo, fmaf(z, c_hi, -K));
}
__device__ __forceinline__ bool fold_ok(float m, float c_hi) {
  return fabsf(m) * c_hi < 4194304.f;
}
__device__ __forceinline__ float ex2(float a) { return __builtin_amdgcn_exp2f(a); }

// Pairwise sum of a unit's terms (fixed order, shared by every pass that recomputes it).
template <int W>
__device__ __forceinline__ float unit_sum(const float (&e)[W]) {
  if constexpr (W == 8) {
    return ((e[0] + e[1]) + (e[2] + e[3])) + ((e[4] + e[5]) + (e[6] + e[7]));
  } else if constexpr (W == 4) {
    return (e[0] + e[1]) + (e[2] + e[3]);
  } else {
    return e[0];
  }
}

// ------------------------------------------------------------------ data shared across workgroups
//
// Values one workgroup hands to another inside a kernel go through device-scope atomic stores
// and loads, which are coherent across the XCDs' separate L2 caches without a cache writeback
// or invalidate.  The writer waits for its stores to complete before it updates an arrival
// counter (a device-scope atomic add); a reader loads them only after its own update of that
// counter has returned the count that makes it the last arrival.
//
// ORDERING ASSUMPTION.  Every hand-off inside a launch uses this protocol and no release or
// acquire fence:
//   writer: relaxed agent-scope atomic stores of the data
//           -> wait_memory() (s_waitcnt 0: every store acknowledged by the device-coherent
//              level; compiler signal fences on both sides keep the compiler from moving
//              memory operations across it)
//           -> __syncthreads() (all of the workgroup's writers have waited)
//           -> one relaxed agent-scope atomic add on the request's counter;
//   reader: its own relaxed atomic on that counter returns the value that makes it the last
//           (or its poll sees the final count) -> __syncthreads() -> relaxed agent-scope
//           atomic loads of the data.
// The HIP memory model gives relaxed atomics no such ordering; the protocol relies on gfx950
// completing a store before acknowledging it and on agent-scope accesses bypassing the
// non-coherent L2, so that an acknowledged store is seen by any later agent-scope load.
// Fences were left out on purpose: on gfx950 an agent-scope release / acquire is a full L2
// writeback / invalidate, measured at ~60 ns of serialised GPU time each, which one fence
// pair per row tile turned into a 12.7x slower stream.  The protocol was run in soak tests
// with the partials poisoned between runs (no wrong or missing merge, counters back to zero).
// The sites that rely on it:
//   - share_store / share_load: the stop rows' chunk sums (stream_chunks -> draw_pick), in
//     k_finish (counter `done`), k_onepass (completion counter) and the accurate redraw (the
//     drawing workgroup reads back its own sums, the same protocol within one workgroup);
//   - put_partial / get_partial and put_u32 / get_rec with SHARED: the row partials and slot
//     records that k_greedy1 and k_onepass hand to the request's last arrival or its waiting
//     tiles (counter `arrive`, the 64-bit arrival word of k_onepass);
//   - the counters' own resets by their last user (k_greedy1, k_onepass), which the next
//     launch reads after the kernel boundary.
// Between two launches (k_rowstats -> k_finish) the kernel boundary orders everything and
// plain accesses suffice.
__device__ __forceinline__ void share_store(double *p, double v) {
  __hip_atomic_store(reinterpret_cast<unsigned long long *>(p),
                     (unsigned long long)__double_as_longlong(v), __ATOMIC_RELAXED,
                     __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ double share_load(const double *p) {
  return __longlong_as_double((long long)__hip_atomic_load(
      reinterpret_cast<unsigned long long *>(const_cast<double *>(p)), __ATOMIC_RELAXED,
      __HIP_MEMORY_SCOPE_AGENT));
}
// Block until every memory operation this thread issued has completed.
__device__ __forceinline__ void wait_memory() {
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
  __builtin_amdgcn_s_waitcnt(0);
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
}

// ------------------------------------------------------------------ wave / block reductions


// Lane moves within the wavefront by DPP (a VALU operand modifier, no LDS crossbar): CTRL
// selects the source lane, ROWS the 16-lane rows that receive it (the others receive 0).
template <int CTRL, int ROWS>
__device__ __forceinline__ double dpp_move(double v) {
  const unsigned long long b = (unsigned long long)__double_as_longlong(v);
  const int lo = __builtin_amdgcn_update_dpp(0, (int)(unsigned)b, CTRL, ROWS, 0xF, false);
  const int hi = __builtin_amdgcn_update_dpp(0, (int)(unsigned)(b >> 32), CTRL, ROWS, 0xF, false);
  return __longlong_as_double((long long)(((unsigned long long)(unsigned)hi << 32) |
                                          (unsigned long long)(unsigned)lo));
}
// Sum over the wavefront (every lane active), returned to every lane: pairs within quads, then
// the half-row and row mirrors give each lane its 16-lane row's sum; the row broadcasts of
// lane 15 (into rows 1 and 3) and lane 31 (into rows 2 and 3) leave the total in lane 63.
__device__ __forceinline__ double wave_sum(double v) {
  v += dpp_move<0xB1, 0xF>(v);   // quad_perm [1, 0, 3, 2]
  v += dpp_move<0x4E, 0xF>(v);   // quad_perm [2, 3, 0, 1]
  v += dpp_move<0x141, 0xF>(v);  // row_half_mirror
  v += dpp_move<0x140, 0xF>(v);  // row_mirror
  v += dpp_move<0x142, 0xA>(v);  // row_bcast:15
  v += dpp_move<0x143, 0xC>(v);  // row_bcast:31
  const unsigned long long b = (unsigned long long)__double_as_longlong(v);
  const unsigned lo = (unsigned)__builtin_amdgcn_readlane((int)(unsigned)b, 63);
  const unsigned hi = (unsigned)__builtin_amdgcn_readlane((int)(unsigned)(b >> 32), 63);
  return __longlong_as_double((long long)(((unsigned long long)hi << 32) | lo));
}

// A lane move that reaches every lane (quad permutations, row rotations): no value to set up
// for lanes that receive nothing.
template <int CTRL>
__device__ __forceinline__ double dpp_all(double v) {
  const unsigned long long b = (unsigned long long)__double_as_longlong(v);
  const int lo = __builtin_amdgcn_mov_dpp((int)(unsigned)b, CTRL, 0xF, 0xF, false);
  const int hi = __builtin_amdgcn_mov_dpp((int)(unsigned)(b >> 32), CTRL, 0xF, 0xF, false);
  return __longlong_as_double((long long)(((unsigned long long)(unsigned)hi << 32) |
                                          (unsigned long long)(unsigned)lo));
}
// Four sums over the wavefront at once (every lane active): v[q] is lane l's term of sum q.
// Two exchange steps transpose them, each lane keeping half of its terms and receiving its
// partner's half of the others (quad partners l ^ 1, then l ^ 2), so lane l then holds one
// sum, q(l) = 2 (l & 1) + ((l >> 1) & 1), over its quad; row rotations by 4 and 8 and the
// exchanges with lanes l ^ 16 and l ^ 32 complete it over the wavefront.  Every lane returns
// the total of sum q(l) (lanes 0..3 hold sums 0, 2, 1, 3).  About a third of the lane moves
// and adds of four wave_sum calls, in a chain of the same depth.
__device__ __forceinline__ double wave_sum4(const double (&v)[4], int lane) {
  const bool b0 = (lane & 1) != 0, b1 = (lane & 2) != 0;
  // step 1: keep sums {2 b0, 2 b0 + 1}, send the other two
  const double s0 = b0 ? v[0] : v[2], s1 = b0 ? v[1] : v[3];
  const double k0 = b0 ? v[2] : v[0], k1 = b0 ? v[3] : v[1];
  const double e0 = k0 + dpp_all<0xB1>(s0);  // quad_perm [1, 0, 3, 2]
  const double e1 = k1 + dpp_all<0xB1>(s1);
  // step 2: keep sum 2 b0 + b1
  const double s = b1 ? e0 : e1, k = b1 ? e1 : e0;
  double f = k + dpp_all<0x4E>(s);  // quad_perm [2, 3, 0, 1]
  f += dpp_all<0x124>(f);           // row_ror:4
  f += dpp_all<0x128>(f);           // row_ror:8
  f += __shfl_xor(f, 16);
  f += __shfl_xor(f, 32);
  return f;
}

// The same reduction pattern for 32-bit values; rows that do not receive a move get `id`,
// the operation's identity.
template <int CTRL, int ROWS>
__device__ __forceinline__ int dpp_move32(int v, int id) {
  return __builtin_amdgcn_update_dpp(id, v, CTRL, ROWS, 0xF, false);
}
__device__ __forceinline__ float wave_max(float v) {
  const int ninf = __float_as_int(-INFINITY);
  v = fmaxf(v, __int_as_float(dpp_move32<0xB1, 0xF>(__float_as_int(v), ninf)));
  v = fmaxf(v, __int_as_float(dpp_move32<0x4E, 0xF>(__float_as_int(v), ninf)));
  v = fmaxf(v, __int_as_float(dpp_move32<0x141, 0xF>(__float_as_int(v), ninf)));
  v = fmaxf(v, __int_as_float(dpp_move32<0x140, 0xF>(__float_as_int(v), ninf)));
  v = fmaxf(v, __int_as_float(dpp_move32<0x142, 0xA>(__float_as_int(v), ninf)));
  v = fmaxf(v, __int_as_float(dpp_move32<0x143, 0xC>(__float_as_int(v), ninf)));
  return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 63));
}
__device__ __forceinline__ int32_t wave_min_i(int32_t v) {
  v = min(v, dpp_move32<0xB1, 0xF>(v, INT32_MAX));
  v = min(v, dpp_move32<0x4E, 0xF>(v, INT32_MAX));
  v = min(v, dpp_move32<0x141, 0xF>(v, INT32_MAX));
  v = min(v, dpp_move32<0x140, 0xF>(v, INT32_MAX));
  v = min(v, dpp_move32<0x142, 0xA>(v, INT32_MAX));
  v = min(v, dpp_move32<0x143, 0xC>(v, INT32_MAX));
  return __builtin_amdgcn_readlane(v, 63);
}
__device__ __forceinline__ void argmax_merge(float &bv, int32_t &bi, float ov, int32_t oi) {
  if (ov > bv || (ov == bv && oi < bi)) {
    bv = ov;
    bi = oi;
  }
}
// Inclusive scan over a wavefront (fp64, lane order).
// (by DPP: row shifts by 1, 2, 4 and 8 give each lane its prefix within its 16-lane row, lanes
// shifted in from outside the row reading 0; the row broadcasts of lanes 15 and 31 then add
// the rows before)
__device__ __forceinline__ double wave_incl_scan(double v) {
  v += dpp_move<0x111, 0xF>(v);  // row_shr:1
  v += dpp_move<0x112, 0xF>(v);  // row_shr:2
  v += dpp_move<0x114, 0xF>(v);  // row_shr:4
  v += dpp_move<0x118, 0xF>(v);  // row_shr:8
  v += dpp_move<0x142, 0xA>(v);  // row_bcast:15
  v += dpp_move<0x143, 0xC>(v);  // row_bcast:31
  return v;
}

// Block reductions with one barrier each.  Every call site owns its LDS array, and the next
// write to that array is separated from these reads by another reduction's barrier.
template <int NW>
__device__ __forceinline__ float block_max1(float v, float *sh) {
  v = wave_max(v);
  if ((threadIdx.x & 63) == 0) sh[threadIdx.x >> 6] = v;
  __syncthreads();
  float r = sh[0];
#pragma unroll
  for (int i = 1; i < NW; ++i) r = fmaxf(r, sh[i]);
  return r;
}
template <int NW>
__device__ __forceinline__ double block_sum1(double v, double *sh) {
  v = wave_sum(v);
  if ((threadIdx.x & 63) == 0) sh[threadIdx.x >> 6] = v;
  __syncthreads();
  double r = sh[0];
#pragma unroll
  for (int i = 1; i < NW; ++i) r += sh[i];
  return r;
}
template <int NW>
__device__ __forceinline__ int32_t block_min1(int32_t v, int32_t *sh) {
  v = wave_min_i(v);
  if ((threadIdx.x & 63) == 0) sh[threadIdx.x >> 6] = v;
  __syncthreads();
  int32_t r = sh[0];
#pragma unroll
  for (int i = 1; i < NW; ++i) r = sh[i] < r ? sh[i] : r;
  return r;
}

// Exclusive scan over the block in thread order (fp64); also returns the block total.
// Ends with a barrier so `sh` can be reused at once.
template <int NW>
__device__ double block_excl_scan(double v, double *sh, double &total) {
  const int w = threadIdx.x >> 6;
  const double inc = wave_incl_scan(v);
  if ((threadIdx.x & 63) == 63) sh[w] = inc;
  __syncthreads();
  double off = 0.0;
  total = 0.0;
#pragma unroll
  for (int i = 0; i < NW; ++i) {
    if (i < w) off += sh[i];
    total += sh[i];
  }
  __syncthreads();
  return off + inc - v;
}

// First / last thread (by id) for which `pred` holds, block-wide: INT32_MAX / -1 if none.
template <int NW>
__device__ int32_t block_first(bool pred, int32_t *sh) {
  const uint64_t m = __ballot(pred);
  if ((threadIdx.x & 63) == 0)
    sh[threadIdx.x >> 6] =
        m ? (int32_t)(threadIdx.x & ~63u) + __ffsll((long long)m) - 1 : INT32_MAX;
  __syncthreads();
  int32_t r = INT32_MAX;
#pragma unroll
  for (int i = 0; i < NW; ++i) r = sh[i] < r ? sh[i] : r;
  __syncthreads();
  return r;
}
template <int NW>
__device__ int32_t block_last(bool pred, int32_t *sh) {
  const uint64_t m = __ballot(pred);
  if ((threadIdx.x & 63) == 0)
    sh[threadIdx.x >> 6] = m ? (int32_t)(threadIdx.x & ~63u) + 63 - __clzll((long long)m) : -1;
  __syncthreads();
  int32_t r = -1;
#pragma unroll
  for (int i = 0; i < NW; ++i) r = sh[i] > r ? sh[i] : r;
  __syncthreads();
  return r;
}

// ------------------------------------------------------------------ row statistics of a tile

struct StatsLds {
  float mx[kRsWaves];
  double sum[kRsWaves];
  int32_t idx[kRsWaves];
};

// Values a workgroup hands to another workgroup of the same launch (the one-launch path) are
// written and read with device-scope atomics (SHARED); between two launches plain accesses
// suffice, the kernel boundary orders them.
template <bool SHARED>
__device__ __forceinline__ void put_partial(Partial *p, const Partial &v) {
  if constexpr (SHARED) {
    const unsigned long long lo = (unsigned long long)__float_as_uint(v.m) |
                                  ((unsigned long long)(uint32_t)v.idx << 32);
    __hip_atomic_store(reinterpret_cast<unsigned long long *>(p), lo, __ATOMIC_RELAXED,
                       __HIP_MEMORY_SCOPE_AGENT);
    share_store(&p->s, v.s);
  } else {
    *p = v;
  }
}
template <bool SHARED>
__device__ __forceinline__ Partial get_partial(const Partial *p) {
  if constexpr (SHARED) {
    const unsigned long long lo =
        __hip_atomic_load(reinterpret_cast<unsigned long long *>(const_cast<Partial *>(p)),
                          __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    Partial v;
    v.m = __uint_as_float((uint32_t)lo);
    v.idx = (int32_t)(uint32_t)(lo >> 32);
    v.s = share_load(&p->s);
    return v;
  } else {
    return *p;
  }
}
template <bool SHARED>
__device__ __forceinline__ void put_u32(void *p, uint32_t v) {
  if constexpr (SHARED)
    __hip_atomic_store(static_cast<uint32_t *>(p), v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  else
    *static_cast<uint32_t *>(p) = v;
}
template <bool SHARED>
__device__ __forceinline__ SlotRec get_rec(const SlotRec *p) {
  if constexpr (SHARED) {
    unsigned long long *q = reinterpret_cast<unsigned long long *>(const_cast<SlotRec *>(p));
    const unsigned long long a = __hip_atomic_load(q, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    const unsigned long long c =
        __hip_atomic_load(q + 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    SlotRec r;
    r.z = __uint_as_float((uint32_t)a);
    r.tok = (int32_t)(uint32_t)(a >> 32);
    r.u = __uint_as_float((uint32_t)c);
    r.pad = 0;
    return r;
  } else {
    return *p;
  }
}

// A row tile's nu units, NV per thread (unit j * kRsThreads + tid), with 16-byte nontemporal
// loads issued together; units past nu hold the filler.
template <int DT, bool VEC, int NV>
__device__ __forceinline__ void load_tile(const typename Unit<DT, VEC>::Store *tile, int32_t nu,
                                          typename Unit<DT, VEC>::Raw (&raw)[NV]) {
  using U = Unit<DT, VEC>;
  const int tid = threadIdx.x;
  if (nu == kRsThreads * NV) {
#pragma unroll
    for (int j = 0; j < NV; ++j) raw[j] = U::template load<true>(tile, j * kRsThreads + tid);
  } else {
#pragma unroll
    for (int j = 0; j < NV; ++j) {
      const int32_t u = j * kRsThreads + tid;
      raw[j] = u < nu ? U::template load<true>(tile, u) : U::filler();
    }
  }
}

// Statistics of the row tile [lo, hi) (nu units, in registers from load_tile) by a workgroup of
// kRsThreads: the tile maximum M, then for a sampled row (T > 0) the sum of 2^((z - M) c) and
// for a greedy row the lowest index holding M, written to `out`.  The logit at `tok`, if the
// tile holds it, goes to `zrec`.  Called by every thread of the workgroup.
template <int DT, bool VEC, int NV, bool SHARED>
__device__ __forceinline__ void tile_stats(const typename Unit<DT, VEC>::Raw (&raw)[NV],
                                           const typename Unit<DT, VEC>::Store *tile,
                                           int32_t nu, int64_t lo, int64_t hi, float T,
                                           int32_t tok, Partial *out, float *zrec,
                                           StatsLds &sh) {
  using U = Unit<DT, VEC>;
  constexpr int W = U::W;
  constexpr int NT = kRsThreads;
  constexpr int NW = kRsWaves;
  const int tid = threadIdx.x;
  const float tm = U::thread_max(raw);
  const float M = block_max1<NW>(tm, sh.mx);

  // The logit at the row's draft token, for the accept tests: written by the thread holding
  // it, in the one tile that does.
  if (tok >= lo && tok < hi) {
    const int32_t off = (int32_t)(tok - lo);
    const int32_t uo = off / W;
    if (uo % NT == tid) {
      float z = 0.f;
#pragma unroll
      for (int j = 0; j < NV; ++j) {
        if (j == uo / NT) {
          float xv[W];
          U::cvt(raw[j], xv);
#pragma unroll
          for (int q = 0; q < W; ++q)
            if (q == off % W) z = xv[q];
        }
      }
      put_u32<SHARED>(zrec, __float_as_uint(z));
    }
  }

  if (T > 0.f && M == -INFINITY) {
    // every logit of the tile masked: no mass (the row has a finite logit elsewhere)
    if (tid == 0) put_partial<SHARED>(out, Partial{M, 0, 0.0});
  } else if (T > 0.f) {
    const TempConst tc = temp_const(T);
    if (fold_ok(M, tc.c_hi) && tc.c < 1e6 && tc.c > 1e-30) {
      // The common case: two-FMA exponent arguments.  In this range of c a filler's
      // argument is -inf or below -200, so its term is exactly 0 and needs no mask.
      const float K = (float)((double)M * tc.c);
      // Unit sums, then a fixed pairwise tree over the thread's NV units in fp32 (at most 64
      // terms of at most ~1.4 each: at most ~6 roundings, 3.6e-7 relative); everything
      // beyond the thread is fp64.
      float us[NV];
#pragma unroll
      for (int j = 0; j < NV; ++j) {
        float x[W], e[W];
        U::cvt(raw[j], x);
#pragma unroll
        for (int q = 0; q < W; ++q) e[q] = ex2(arg_folded(x[q], K, tc.c_hi, tc.c_lo));
        us[j] = unit_sum<W>(e);
      }
#pragma unroll
      for (int st = 1; st < NV; st *= 2) {
#pragma unroll
        for (int j = 0; j + st < NV; j += 2 * st) us[j] += us[j + st];
      }
      const double S = block_sum1<NW>((double)us[0], sh.sum);
      // to the shifted form, sum 2^((z - M) c): factor 2^(K - M c), one rounding
      if (tid == 0)
        put_partial<SHARED>(out, Partial{M, 0, S * exp2(fma(-(double)M, tc.c, (double)K))});
    } else {
      // Extreme temperatures or logits: overflow-safe arguments, units re-read one at a time
      // (cache hits) to keep this rare path out of the common path's registers.
      double acc = 0.0;
#pragma unroll 1
      for (int j = 0; j < NV; ++j) {
        const int32_t u = j * NT + tid;
        if (u < nu) {
          float x[W], e[W];
          U::cvt(U::template load<false>(tile, u), x);
#pragma unroll
          for (int q = 0; q < W; ++q) e[q] = ex2(arg_shifted(x[q], M, tc.c_hi, tc.c_lo));
          acc += (double)unit_sum<W>(e);
        }
      }
      const double S = block_sum1<NW>(acc, sh.sum);
      if (tid == 0) put_partial<SHARED>(out, Partial{M, 0, S});
    }
  } else {
    // Greedy row: the lowest index holding the tile maximum; only threads whose own maximum
    // equals it search their units.
    int32_t ti = INT32_MAX;
    if (tm == M) {
#pragma unroll
      for (int j = 0; j < NV; ++j) {
        float x[W];
        U::cvt(raw[j], x);
        const int32_t u = j * NT + tid;
#pragma unroll
        for (int q = 0; q < W; ++q)
          if (ti == INT32_MAX && u < nu && x[q] == M) ti = (int32_t)((lo / W + u) * W + q);
      }
    }
    const int32_t bi = block_min1<NW>(ti, sh.idx);
    if (tid == 0) put_partial<SHARED>(out, Partial{M, bi, 0.0});
  }
}

// ------------------------------------------------------------------ k_rowstats

// One workgroup per (row slot, tile): blockIdx.x is the tile of the row, blockIdx.y +
// blockIdx.z * gridDim.y the row slot (request * spr + slot).  Slots beyond a request's rows
// (gamma_b < gamma, or draft rows of a greedy request) exit at once.
template <int DT, bool VEC>
__global__ __launch_bounds__(kRsThreads) void k_rowstats(Params P) {
  using U = Unit<DT, VEC>;
  using Store = typename U::Store;
  constexpr int W = U::W;
  constexpr int NV = int(kTileElems / kRsThreads) / W;  // units per thread
  __shared__ StatsLds sh;
  const int tid = threadIdx.x;
  const uint32_t slot = blockIdx.y + blockIdx.z * gridDim.y;
  const uint32_t spr = (uint32_t)P.spr;
  if (slot >= (uint32_t)P.B * spr) return;
  const int32_t b = (int32_t)(slot / spr);
  const int32_t k = (int32_t)(slot - (uint32_t)b * spr);
  int64_t dbase;
  int32_t gb;
  float T;
  request(P, b, dbase, gb, T);
  const void *base;
  int64_t row;
  int32_t pos;  // draft position whose token this row is tested at; gb for the bonus row
  if (k <= P.gamma) {
    if (k > gb) return;
    base = P.target;
    row = dbase + b + k;
    pos = k;
  } else {
    const int32_t i = k - P.gamma - 1;
    if (i >= gb || !(T > 0.f)) return;
    base = P.draft;
    row = dbase + i;
    pos = i;
  }
  const int32_t xtok = pos < gb ? P.tokens[dbase + pos] : -1;
  if (k <= P.gamma && pos < gb && blockIdx.x == 0 && tid == 0) {
    P.rec[slot].tok = xtok;
    P.rec[slot].u = T > 0.f ? P.uniforms[2 * (dbase + b + pos)] : 0.f;
  }
  // k_finish counts its workgroups per request from zero: the first tile of the request's
  // first target row (present in every request) clears the counter for it.
  if (k == 0 && blockIdx.x == 0 && threadIdx.x == 0) P.done[b * kCounterStride] = 0u;
  const int64_t lo = (int64_t)blockIdx.x * P.split_len;
  const int64_t hi = lo + P.split_len < P.V ? lo + P.split_len : P.V;
  const Store *tile = static_cast<const Store *>(row_ptr<DT>(base, row, P.V)) + lo / W;
  const int32_t nu = (int32_t)((hi - lo + W - 1) / W);
  typename U::Raw raw[NV];
  load_tile<DT, VEC, NV>(tile, nu, raw);
  tile_stats<DT, VEC, NV, false>(raw, tile, nu, lo, hi, T, T > 0.f ? xtok : -1,
                                 P.parts + (int64_t)slot * P.nsplit + blockIdx.x, &P.rec[slot].z,
                                 sh);
}

// ------------------------------------------------------------------ finishing a request

// Residual weight of one element of the stop row, scaled by S_t:
//   residual mode: S_t (p_k - q_k)_+ = (e_t - rho e_d)_+ with rho = S_t / S_d (two-float);
//   bonus mode:    S_t p_k = e_t.
template <int W>
__device__ __forceinline__ void resid_weights(const float (&zt)[W], const float (&zd)[W],
                                              const Stop &st, float (&r)[W]) {
#pragma unroll
  for (int q = 0; q < W; ++q) {
    const float et = ex2(arg_shifted(zt[q], st.mt, st.c_hi, st.c_lo));
    if (st.mode == kModeResidual) {
      const float ed = ex2(arg_shifted(zd[q], st.md, st.c_hi, st.c_lo));
      const float v = fmaf(-ed, st.rho_lo, fmaf(-ed, st.rho_hi, et));
      r[q] = v > 0.f ? v : 0.f;
    } else {
      r[q] = et;
    }
  }
}

// Weights and pairwise sum of unit u of the stop row(s).
template <int DT, bool VEC>
__device__ __forceinline__ float resid_unit(const typename Unit<DT, VEC>::Store *tr,
                                            const typename Unit<DT, VEC>::Store *dr, int64_t u,
                                            const Stop &st, float (&r)[Unit<DT, VEC>::W]) {
  using U = Unit<DT, VEC>;
  constexpr int W = U::W;
  float zt[W], zd[W];
  U::cvt(U::template load<false>(tr, u), zt);
  if (st.mode == kModeResidual) {
    U::cvt(U::template load<false>(dr, u), zd);
  } else {
#pragma unroll
    for (int q = 0; q < W; ++q) zd[q] = 0.f;
  }
  resid_weights<W>(zt, zd, st, r);
  return unit_sum<W>(r);
}

// Residual weights of a stop row whose residual is small, without forming p - q: for
// delta_k = log2(q_k / p_k) = (zd_k - zt_k) c + kd (kd: the maxima's and normalisers' part,
// folded into one float), S_t (p_k - q_k) = e_t,k (1 - 2^delta_k), and where |delta| < 1 the
// factor 1 - 2^delta is taken by expm1, so the term keeps its relative accuracy however close
// q_k is to p_k (the logit difference is exact, or correctly rounded, in fp32, and delta is
// small exactly when the term is).  Elsewhere the term is e_t,k - 2^(a_k + delta_k), a_k the
// exponent argument of e_t,k, which cannot overflow.  A masked target entry (e_t = 0) gives 0.
constexpr float kLn2f = 0.69314718055994531f;
__device__ __forceinline__ float acc_term(float zt, float zd, const Stop &st, float kd,
                                          float &et) {
  const float a = arg_shifted(zt, st.mt, st.c_hi, st.c_lo);
  et = ex2(a);
  const float dz = zd - zt;
  const float dl = fmaf(dz, st.c_hi, fmaf(dz, st.c_lo, kd));
  if (!(et > 0.f)) return 0.f;
  if (fabsf(dl) < 1.f) return -et * expm1f(dl * kLn2f);
  return et - ex2(a + dl);
}
template <int W>
__device__ __forceinline__ void resid_weights_acc(const float (&zt)[W], const float (&zd)[W],
                                                  const Stop &st, float kd, float (&r)[W]) {
#pragma unroll
  for (int q = 0; q < W; ++q) {
    float et;
    const float v = acc_term(zt[q], zd[q], st, kd, et);
    r[q] = v > 0.f ? v : 0.f;
  }
}

// Weights and pairwise sum of unit u of the stop row(s): the ordinary form, or (ACC) the
// relatively accurate one of a small residual.
template <int DT, bool VEC, bool ACC>
__device__ __forceinline__ float unit_weights(const typename Unit<DT, VEC>::Store *tr,
                                              const typename Unit<DT, VEC>::Store *dr, int64_t u,
                                              const Stop &st, float kd,
                                              float (&r)[Unit<DT, VEC>::W]) {
  using U = Unit<DT, VEC>;
  constexpr int W = U::W;
  if constexpr (!ACC) {
    return resid_unit<DT, VEC>(tr, dr, u, st, r);
  } else {
    float zt[W], zd[W];
    U::cvt(U::template load<false>(tr, u), zt);
    U::cvt(U::template load<false>(dr, u), zd);
    resid_weights_acc<W>(zt, zd, st, kd, r);
    return unit_sum<W>(r);
  }
}

// Draw from p over a whole target row (used only when the residual is empty after rounding).
template <int DT, int NT>
__device__ int32_t draw_from_row(const void *tr, int64_t V, const Stop &st, double u,
                                 double *shd, int32_t *shi, double &total) {
  constexpr int NW = NT / 64;
  const int tid = threadIdx.x;
  const int64_t per = (V + NT - 1) / NT;
  const int64_t a = tid * per;
  const int64_t e_ = a + per < V ? a + per : V;
  double mine = 0.0;
  for (int64_t k = a; k < e_; ++k)
    mine += (double)ex2(arg_shifted(logit_at<DT>(tr, k), st.mt, st.c_hi, st.c_lo));
  const double before = block_excl_scan<NW>(mine, shd, total);
  const double target = u * total;
  const int32_t first = block_first<NW>(mine > 0.0 && before + mine > target, shi);
  const int32_t last = block_last<NW>(mine > 0.0, shi);
  const int32_t pick = first != INT32_MAX ? first : last;
  int32_t tok = -1;
  if (tid == pick) {
    double run = before;
    int32_t lastpos = -1;
    for (int64_t k = a; k < e_; ++k) {
      const float e = ex2(arg_shifted(logit_at<DT>(tr, k), st.mt, st.c_hi, st.c_lo));
      run += (double)e;
      if (e > 0.f) {
        lastpos = (int32_t)k;
        if (first != INT32_MAX && run > target) {
          tok = (int32_t)k;
          break;
        }
      }
    }
    if (tok < 0) tok = lastpos;
  }
  return tok;
}

// Merged rows of one request, in LDS.
struct ReqLds {
  float m[2 * SPEC_MAX_GAMMA + 1];   // row maxima by row slot: target rows 0..gamma, then drafts
  double s[2 * SPEC_MAX_GAMMA + 1];  // row sums (sampled requests)
  int32_t i[SPEC_MAX_GAMMA + 1];     // target argmax (greedy requests)
  int32_t j;                         // the stop row
};

// Steps 1 and 2 of finishing request b, for a workgroup of NT threads:
//  1. merge the row partials (a group of lanes per row slot, one lane per tile, fp64);
//  2. accept tests lane-parallel on wavefront 0 (p(x), q(x) in fp64 from the logits that
//     k_rowstats captured) and the first rejection by ballot + find-first-set.
// Merged rows sit in L by row slot (target row r at r, draft row i at gamma + 1 + i).  With
// `write`, the outputs and the row probes are written.  Ends with a barrier; the stop row is
// in L.j.  Returns the request's temperature constant.  SHARED: the partials and slot records
// were written by other workgroups of the same launch.
template <int NT, bool SHARED>
__device__ __forceinline__ TempConst finish_head(const Params &P, int32_t b, bool write, ReqLds &L,
                                 int64_t &dbase, int32_t &gb, bool &sampling) {
  constexpr int NW = NT / 64;
  constexpr int G = 4;  // rounds of row slots whose partials are loaded at once
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int64_t slot0 = (int64_t)b * P.spr;
  const int32_t dslot = P.gamma + 1;  // slot of draft row 0

  // Row slots are merged in lane groups: LP lanes per slot (the smallest power of two >= the
  // tiles per row, at most 64), R = 64 / LP slots per wavefront at a time; lane l of a group
  // holds tiles l, l + LP, ... of its slot.
  int32_t lp = 1;
  while (lp < P.nsplit && lp < 64) lp <<= 1;
  const int32_t R = 64 / lp;
  const int32_t grp = lane / lp, sl = lane - grp * lp;
  const int32_t per_round = NW * R;  // slots merged per round by the workgroup

  // One round trip carries everything: the request's bounds and temperature, the partials
  // of its row slots (up to G rounds), and the slot records (logits at the draft tokens, the
  // tokens, their uniforms) that k_rowstats left.
  float T;
  request(P, b, dbase, gb, T);
  SlotRec rt = {};
  float zd = 0.f;
  if (wave == 0 && lane < P.gamma) {
    rt = get_rec<SHARED>(P.rec + slot0 + lane);
    if (!P.greedy_all) zd = get_rec<SHARED>(P.rec + slot0 + dslot + lane).z;
  }
  Partial pv[G];
#pragma unroll
  for (int q = 0; q < G; ++q) {
    const int32_t k = q * per_round + wave * R + grp;
    pv[q].m = -INFINITY;
    pv[q].idx = INT32_MAX;
    pv[q].s = 0.0;
    if (k < P.spr && sl < P.nsplit)
      pv[q] = get_partial<SHARED>(P.parts + (slot0 + k) * P.nsplit + sl);
  }
  sampling = T > 0.f;
  const int64_t tbase = dbase + b;
  const TempConst tc = temp_const(sampling ? T : 1.f);
  const int32_t x = lane < gb ? rt.tok : -1;
  const float ux = rt.u, zt = rt.z;

  // 1. Merge: maximum, then the sum with each tile's shift taken out in fp64 (sampled), or
  // the lowest-index argmax (greedy), reduced over the lane group.
  for (int32_t r0 = 0; r0 < P.spr; r0 += G * per_round) {
    if (r0 > 0) {
#pragma unroll
      for (int q = 0; q < G; ++q) {
        const int32_t k = r0 + q * per_round + wave * R + grp;
        pv[q].m = -INFINITY;
        pv[q].idx = INT32_MAX;
        pv[q].s = 0.0;
        if (k < P.spr && sl < P.nsplit)
          pv[q] = get_partial<SHARED>(P.parts + (slot0 + k) * P.nsplit + sl);
      }
    }
#pragma unroll
    for (int q = 0; q < G; ++q) {
      if (r0 + q * per_round >= P.spr) break;  // uniform across the workgroup
      const int32_t k = r0 + q * per_round + wave * R + grp;
      const bool live = k < P.spr && (k < dslot ? k <= gb : sampling && k - dslot < gb);
      const Partial *rowp = P.parts + (slot0 + (k < P.spr ? k : 0)) * P.nsplit;
      if (sampling) {
        float m = live ? pv[q].m : -INFINITY;
        if (live)
          for (int32_t p = sl + lp; p < P.nsplit; p += lp)
            m = fmaxf(m, get_partial<SHARED>(rowp + p).m);
        for (int o = lp >> 1; o > 0; o >>= 1) m = fmaxf(m, __shfl_xor(m, o));
        const float M = m;
        double f = 0.0;
        if (live) {
          if (pv[q].m != -INFINITY) f = pv[q].s * exp2(((double)pv[q].m - (double)M) * tc.c);
          for (int32_t p = sl + lp; p < P.nsplit; p += lp) {
            const Partial o = get_partial<SHARED>(rowp + p);
            if (o.m != -INFINITY) f += o.s * exp2(((double)o.m - (double)M) * tc.c);
          }
        }
        for (int o = lp >> 1; o > 0; o >>= 1) f += __shfl_xor(f, o);
        if (live && sl == 0) {
          L.m[k] = M;
          L.s[k] = f;
        }
      } else {
        float bv = live ? pv[q].m : -INFINITY;
        int32_t bi = live ? pv[q].idx : INT32_MAX;
        if (live)
          for (int32_t p = sl + lp; p < P.nsplit; p += lp) {
            const Partial o = get_partial<SHARED>(rowp + p);
            argmax_merge(bv, bi, o.m, o.idx);
          }
        for (int o = lp >> 1; o > 0; o >>= 1) {
          const float ov = __shfl_xor(bv, o);
          const int32_t oi = __shfl_xor(bi, o);
          argmax_merge(bv, bi, ov, oi);
        }
        if (live && sl == 0) {
          L.m[k] = bv;
          L.i[k] = bi;
        }
      }
    }
  }
  __syncthreads();

  // 2. Lane i = draft position i.
  if (wave == 0) {
    bool accept = false;
    double p = 0.0, q = 0.0;
    if (lane < gb) {
      if (!sampling) {
        accept = x == L.i[lane];
      } else {
        if (x >= 0 && x < P.V) {
          p = exp2(((double)zt - (double)L.m[lane]) * tc.c) / L.s[lane];
          q = exp2(((double)zd - (double)L.m[dslot + lane]) * tc.c) / L.s[dslot + lane];
        }
        accept = (double)ux * q < p;
      }
    }
    const uint64_t acc_mask = __ballot(accept);
    const uint64_t valid = gb >= 64 ? ~0ull : ((1ull << gb) - 1ull);
    const uint64_t rej = ~acc_mask & valid;
    const int32_t j = rej ? (int32_t)(__ffsll((long long)rej) - 1) : gb;
    if (lane == 0) L.j = j;
    if (write) {
      if (lane < gb && lane != j) P.out_tokens[tbase + lane] = lane < j ? x : -1;
      if (lane == 0) {
        if (j < gb) P.out_tokens[tbase + gb] = -1;
        if (!sampling) P.out_tokens[tbase + j] = L.i[j];
        P.out_n[b] = j;
      }
      if (sampling && lane < gb) {
        if (P.p_x) P.p_x[dbase + lane] = p;
        if (P.q_x) P.q_x[dbase + lane] = q;
      }
    }
  }
  if (write) {
    for (int32_t r = tid; r <= gb; r += NT) {
      if (P.row_max_t) P.row_max_t[tbase + r] = L.m[r];
      if (sampling && P.row_sum_t) P.row_sum_t[tbase + r] = L.s[r];
    }
    if (sampling) {
      for (int32_t r = tid; r < gb; r += NT) {
        if (P.row_max_d) P.row_max_d[dbase + r] = L.m[dslot + r];
        if (P.row_sum_d) P.row_sum_d[dbase + r] = L.s[dslot + r];
      }
    }
  }
  __syncthreads();
  return tc;
}

// The residual weights' constants for stop row j of a sampled request.
__device__ __forceinline__ Stop make_stop(const ReqLds &L, int32_t gb, int32_t dslot,
                                          const TempConst &tc, int64_t trow, int64_t drow) {
  const int32_t j = L.j;
  Stop st = {};
  st.mode = j < gb ? kModeResidual : kModeBonus;
  st.mt = L.m[j];
  st.st = L.s[j];
  st.c_hi = tc.c_hi;
  st.c_lo = tc.c_lo;
  if (j < gb) {
    st.md = L.m[dslot + j];
    const double rho = L.s[j] / L.s[dslot + j];
    st.rho_hi = (float)rho;
    st.rho_lo = (float)(rho - (double)st.rho_hi);
  }
  st.trow = trow;
  st.drow = drow;
  return st;
}

// Step 3: units [ub, ub_end) of the stop row(s), NT * RU units per pass with all loads of a
// pass in flight (ordinary loads: nontemporal ones here measured a slower row-statistics stream
// in the next call); one fp64 sum per 64-unit chunk (one wavefront-wide load) into cs.  ub is a
// multiple of 64 units, so every chunk is summed by one wavefront.
template <int DT, bool VEC, int NT, int RU, bool ACC = false>
__device__ __forceinline__ void stream_chunks(const Params &P, const Stop &st, int64_t ub,
                                              int64_t ub_end, double *cs, float kd = 0.f) {
  using U = Unit<DT, VEC>;
  using Store = typename U::Store;
  constexpr int W = U::W;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const Store *tr = static_cast<const Store *>(row_ptr<DT>(P.target, st.trow, P.V));
  const Store *dr = static_cast<const Store *>(row_ptr<DT>(P.draft, st.drow, P.V));
  const bool resid = st.mode == kModeResidual;
  for (; ub < ub_end; ub += (int64_t)NT * RU) {
    typename U::Raw rt[RU], rd[RU];
#pragma unroll
    for (int q = 0; q < RU; ++q) {
      const int64_t u = ub + q * NT + tid;
      rt[q] = u < ub_end ? U::template load<false>(tr, u) : U::filler();
      rd[q] = resid && u < ub_end ? U::template load<false>(dr, u) : U::filler();
    }
    if constexpr (RU == 4) {
      // the pass's four chunks reduced together; lane q(l) < 4 stores chunk q(l)'s sum
      double d[4];
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int64_t c0 = ub + q * NT + wave * 64;  // first unit of this chunk
        d[q] = 0.0;
        if (c0 < ub_end) {  // uniform across the wavefront
          float zt[W], zd[W], r[W];
          U::cvt(rt[q], zt);
          U::cvt(rd[q], zd);
          if constexpr (ACC)
            resid_weights_acc<W>(zt, zd, st, kd, r);
          else
            resid_weights<W>(zt, zd, st, r);
          const float us = unit_sum<W>(r);
          d[q] = c0 + lane < ub_end ? (double)us : 0.0;
        }
      }
      const double sum = wave_sum4(d, lane);
      if (lane < 4) {
        const int q = 2 * (lane & 1) + ((lane >> 1) & 1);
        const int64_t c0 = ub + q * NT + wave * 64;
        if (c0 < ub_end) share_store(&cs[c0 / kChunkUnits], sum);
      }
    } else {
#pragma unroll
      for (int q = 0; q < RU; ++q) {
        const int64_t c0 = ub + q * NT + wave * 64;  // first unit of this chunk
        if (c0 >= ub_end) break;  // uniform across the wavefront
        float zt[W], zd[W], r[W];
        U::cvt(rt[q], zt);
        U::cvt(rd[q], zd);
        if constexpr (ACC)
          resid_weights_acc<W>(zt, zd, st, kd, r);
        else
          resid_weights<W>(zt, zd, st, r);
        const float us = unit_sum<W>(r);
        const double sum = wave_sum(c0 + lane < ub_end ? (double)us : 0.0);
        if (lane == 0) share_store(&cs[c0 / kChunkUnits], sum);
      }
    }
  }
}

// LDS of the draw.
template <int NW>
struct DrawLds {
  double shd[NW];
  double acc[2][NW];
  int32_t shi[NW];
  int32_t c, tok;
  double local;
};

// Below this residual mass (relative to the row's normaliser) the draw is recomputed in the
// accurate form.  The ordinary weights (e_t - rho e_d)_+ carry the error of rho = S_t / S_d,
// whose two fp32-term normalisers are each within ~2e-7 relative: an absolute error of at most
// ~3e-7 in the mass and of ~3e-7 / R in the draw's normalised running sum.  Above 0.05 that is
// within 1e-5 relative for the mass and a few 1e-6 at worst (~1e-7 typically) for the draw.
constexpr double kAccurateBelow = 0.05;
constexpr int kAccRU = 2;

// Pick the token from the chunk sums cs of the stop row(s), by a workgroup of NT threads: a
// block scan over the chunk sums picks the chunk holding u * R, a wavefront scan over its 64
// units picks the unit, and a walk over the unit's elements gives the token (into D.tok, -1 if
// every weight is 0).  R: the total.  The chunk sums
// were written by other workgroups (or this one), so they are read with device-scope loads.
template <int DT, bool VEC, int NT, bool ACC>
__device__ void draw_pick(const Params &P, const Stop &st, float kd, const double *cs,
                          double u, DrawLds<NT / 64> &D, double &R) {
  using U = Unit<DT, VEC>;
  using Store = typename U::Store;
  constexpr int W = U::W;
  constexpr int NW = NT / 64;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const Store *tr = static_cast<const Store *>(row_ptr<DT>(P.target, st.trow, P.V));
  const Store *dr = static_cast<const Store *>(row_ptr<DT>(P.draft, st.drow, P.V));
  const int64_t nunits = (P.V + W - 1) / W;
  const int64_t nchunks = (nunits + 63) / 64;

  // Each thread sums a contiguous run of chunks, a block scan places the runs, and the
  // thread whose run crosses the target walks it.  Runs of up to kDrawKeep chunks (every
  // vocabulary up to 128K units) stay in registers, so the walk needs no second round trip.
  constexpr int kDrawKeep = 8;
  const int64_t per = (nchunks + NT - 1) / NT;
  const int64_t a = tid * per;
  const int64_t e_ = a + per < nchunks ? a + per : nchunks;
  const bool kept = per <= kDrawKeep;  // uniform
  double keep[kDrawKeep];
  double mine = 0.0;
  if (kept) {
#pragma unroll
    for (int i = 0; i < kDrawKeep; ++i) keep[i] = a + i < e_ ? share_load(&cs[a + i]) : 0.0;
#pragma unroll
    for (int i = 0; i < kDrawKeep; ++i) mine += keep[i];
  } else {
    for (int64_t c = a; c < e_; ++c) mine += share_load(&cs[c]);
  }
  const double before = block_excl_scan<NW>(mine, D.shd, R);
  const double target = u * R;
  const int32_t first = block_first<NW>(mine > 0.0 && before + mine > target, D.shi);
  const int32_t lastt = block_last<NW>(mine > 0.0, D.shi);
  if (tid == 0) {
    D.c = -1;
    D.tok = -1;
  }
  __syncthreads();
  const int32_t pick = first != INT32_MAX ? first : lastt;
  if (tid == pick) {
    double run = before;
    int64_t lastpos = -1;
    bool found = false;
    if (kept) {
#pragma unroll
      for (int i = 0; i < kDrawKeep; ++i) {
        const double v = keep[i];
        if (!found && a + i < e_) {
          if (v > 0.0) {
            lastpos = a + i;
            if (first != INT32_MAX && run + v > target) {
              D.c = (int32_t)(a + i);
              D.local = target - run;
              found = true;
            }
          }
          run += v;
        }
      }
    } else {
      for (int64_t c = a; c < e_; ++c) {
        const double v = share_load(&cs[c]);
        if (v > 0.0) {
          lastpos = c;
          if (first != INT32_MAX && run + v > target) {
            D.c = (int32_t)c;
            D.local = target - run;
            break;
          }
        }
        run += v;
      }
    }
    if (D.c < 0) {
      D.c = (int32_t)lastpos;
      D.local = INFINITY;
    }
  }
  __syncthreads();
  const int32_t csel = D.c;
  if (csel >= 0 && wave == 0) {
    // The chunk's 64 units: a wavefront scan picks the unit, its lane walks the elements.
    // With no crossing (u at the far end), the last unit with mass is taken.
    const int64_t uu = (int64_t)csel * 64 + lane;
    float r[W];
    float us = 0.f;
    if (uu < nunits) us = unit_weights<DT, VEC, ACC>(tr, dr, uu, st, kd, r);
    const double local = D.local;
    const double incl = wave_incl_scan((double)us);
    const uint64_t cross = __ballot(us > 0.f && incl > local);
    const uint64_t pos = __ballot(us > 0.f);
    const int32_t pl = cross ? __ffsll((long long)cross) - 1
                             : (pos ? 63 - __clzll((long long)pos) : -1);
    if (lane == pl) {
      double run = incl - (double)us;
      int32_t tok = -1, lastpos = -1;
      for (int e = 0; e < W; ++e) {
        if (r[e] > 0.f) {
          lastpos = (int32_t)(uu * W + e);
          run += (double)r[e];
          if (cross && tok < 0 && run > local) tok = lastpos;
        }
      }
      D.tok = tok >= 0 ? tok : lastpos;
    }
  }
  __syncthreads();
}

// Normaliser sums of the stop row(s) in the accurate form, over the whole row by one
// workgroup: St = sum e_t,k and Dd = sum e_t,k (1 - 2^delta0_k), delta0_k = (zd - zt) c + kd0
// = log2(e_d,k / e_t,k), so that S_d (in e_t's shift) is St - Dd with Dd as accurate as its
// terms.
template <int DT, bool VEC, int NT, int RU>
__device__ void accurate_sums(const Params &P, const Stop &st, float kd0, DrawLds<NT / 64> &D,
                              double &St, double &Dd) {
  using U = Unit<DT, VEC>;
  using Store = typename U::Store;
  constexpr int W = U::W;
  constexpr int NW = NT / 64;
  const int tid = threadIdx.x;
  const Store *tr = static_cast<const Store *>(row_ptr<DT>(P.target, st.trow, P.V));
  const Store *dr = static_cast<const Store *>(row_ptr<DT>(P.draft, st.drow, P.V));
  const int64_t nunits = (P.V + W - 1) / W;
  double s_t = 0.0, s_d = 0.0;
  for (int64_t ub = 0; ub < nunits; ub += (int64_t)NT * RU) {
    typename U::Raw rt[RU], rd[RU];
#pragma unroll
    for (int q = 0; q < RU; ++q) {
      const int64_t u = ub + q * NT + tid;
      rt[q] = u < nunits ? U::template load<false>(tr, u) : U::filler();
      rd[q] = u < nunits ? U::template load<false>(dr, u) : U::filler();
    }
#pragma unroll
    for (int q = 0; q < RU; ++q) {
      float zt[W], zd[W], et[W], gt[W];
      U::cvt(rt[q], zt);
      U::cvt(rd[q], zd);
#pragma unroll
      for (int k = 0; k < W; ++k) gt[k] = acc_term(zt[k], zd[k], st, kd0, et[k]);
      s_t += (double)unit_sum<W>(et);
      s_d += (double)unit_sum<W>(gt);
    }
  }
  St = block_sum1<NW>(s_t, D.acc[0]);
  Dd = block_sum1<NW>(s_d, D.acc[1]);
}

// Step 4, the draw, by a workgroup of NT threads once every chunk sum of request b is in cs.
// A residual whose mass is small is drawn again in the accurate form: normalisers from the stop
// rows' own terms, then chunk sums of the accurate weights written over cs, then the same
// pick.
template <int DT, bool VEC, int NT>
__device__ __forceinline__ void draw_token(const Params &P, int32_t b, const Stop &st, double *cs,
                                           DrawLds<NT / 64> &D) {
  using U = Unit<DT, VEC>;
  constexpr int W = U::W;
  const double u = (double)P.uniforms[2 * st.trow + 1];
  double R;
  draw_pick<DT, VEC, NT, false>(P, st, 0.f, cs, u, D, R);
  double norm = st.st;  // the normaliser R is divided by for the probe
  if (st.mode == kModeResidual && R < kAccurateBelow * st.st) {
    // log2(e_d / e_t) = (zd - zt) c + kd0, kd0 = -(md - mt) c
    const double c = (double)st.c_hi + (double)st.c_lo;
    const double kd0 = -((double)st.md - (double)st.mt) * c;
    double St, Dd;
    // (kAccRU units per thread and pass: this rare path must not raise the kernel's registers)
    accurate_sums<DT, VEC, NT, kAccRU>(P, st, (float)kd0, D, St, Dd);
    // delta_k = log2(q_k / p_k) = log2(e_d,k / e_t,k) + log2(S_t / S_d), S_d = St - Dd
    const double kd = kd0 - log1p(-Dd / St) / 0.69314718055994531;
    stream_chunks<DT, VEC, NT, kAccRU, true>(P, st, 0, (P.V + W - 1) / W, cs, (float)kd);
    wait_memory();
    __syncthreads();
    draw_pick<DT, VEC, NT, true>(P, st, (float)kd, cs, u, D, R);
    norm = St;
  }
  if (D.tok >= 0) {
    if (threadIdx.x == 0) {
      P.out_tokens[st.trow] = D.tok;
      if (P.resid_mass) P.resid_mass[b] = R / norm;
    }
  } else {
    // Empty residual after rounding: fall back to a draw from p_j.
    Stop sp = st;
    sp.mode = kModeBonus;
    double tot;
    const int32_t tok = draw_from_row<DT, NT>(row_ptr<DT>(P.target, st.trow, P.V), P.V, sp, u,
                                              D.shd, D.shi, tot);
    if (tok >= 0) D.tok = tok;
    __syncthreads();
    if (threadIdx.x == 0) {
      P.out_tokens[st.trow] = D.tok;
      if (P.resid_mass) P.resid_mass[b] = tot / st.st;
    }
  }
}

// ------------------------------------------------------------------ k_finish

// Workgroups (slice, request), in an XCD-aware order: blockIdx.x = 8 * slice + x and group
// g = blockIdx.y + blockIdx.z * gridDim.y give request 8 g + x.  Workgroups go to the eight
// XCDs round-robin by linear id, and gridDim.x is a multiple of 8, so every slice of a request
// runs on one XCD and the draw finds the stop rows its slices read in that XCD's L2 (measured:
// workload 3's finish 0.2 us faster; placement changes only speed, never results).  Every
// workgroup of a sampled request repeats steps 1-2
// (a few KB of partials, cheaper than another launch); slice 0 writes the outputs.  Then each
// streams its slice of the stop row(s) (step 3), publishes its chunk sums and counts itself
// in; the last one draws (step 4).  Greedy requests finish in slice 0 after step 2.
template <int DT, bool VEC>
__global__ __launch_bounds__(kThreads) void k_finish(Params P) {
  constexpr int W = Unit<DT, VEC>::W;
  __shared__ ReqLds L;
  __shared__ DrawLds<kWaves> D;
  __shared__ int32_t s_last;
  const uint32_t b32 = (blockIdx.y + blockIdx.z * gridDim.y) * 8u + (blockIdx.x & 7u);
  if (b32 >= (uint32_t)P.B) return;
  const int32_t b = (int32_t)b32;
  const int32_t split = (int32_t)(blockIdx.x >> 3);
  if (split != 0 && (P.greedy_all || !(P.temps[b] > 0.f))) return;
  int64_t dbase;
  int32_t gb;
  bool sampling;
  const TempConst tc = finish_head<kThreads, false>(P, b, split == 0, L, dbase, gb, sampling);
  if (!sampling) return;
  const Stop st = make_stop(L, gb, P.gamma + 1, tc, dbase + b + L.j, dbase + L.j);
  const int64_t nunits = (P.V + W - 1) / W;
  const int64_t ub = (int64_t)split * P.slice_units;
  const int64_t ue = ub + P.slice_units < nunits ? ub + P.slice_units : nunits;
  double *cs = P.chunk_sums + (int64_t)b * P.chunk_stride;
  stream_chunks<DT, VEC, kThreads, kFinRU>(P, st, ub, ue, cs);
  wait_memory();
  __syncthreads();
  if (threadIdx.x == 0)
    s_last = __hip_atomic_fetch_add(&P.done[b * kCounterStride], 1u, __ATOMIC_RELAXED,
                                    __HIP_MEMORY_SCOPE_AGENT) ==
             (uint32_t)P.nslice - 1u;
  __syncthreads();
  if (!s_last) return;
  draw_token<DT, VEC, kThreads>(P, b, st, cs, D);
}

// ------------------------------------------------------------------ k_greedy1

// A greedy call (spec_verify_greedy) in one launch.  Workgroups (tile, row slot) as k_rowstats,
// target rows only.  Each hands its (max, lowest argmax) partial over with device-scope atomic
// stores, waits for them to complete and adds itself to its request's arrival counter; the
// last arrival of a request merges the request's partials and writes its outputs, as k_finish's
// slice 0 does.  No workgroup waits for another, so any grid works; the last arrival returns
// the counter to zero.
template <int DT, bool VEC>
__global__ __launch_bounds__(kRsThreads) void k_greedy1(Params P) {
  using U = Unit<DT, VEC>;
  using Store = typename U::Store;
  constexpr int W = U::W;
  constexpr int NV = int(kTileElems / kRsThreads) / W;
  __shared__ StatsLds sh;
  __shared__ ReqLds L;
  __shared__ int32_t s_last;
  const int tid = threadIdx.x;
  const uint32_t slot = blockIdx.y + blockIdx.z * gridDim.y;
  const uint32_t spr = (uint32_t)P.spr;
  if (slot >= (uint32_t)P.B * spr) return;
  const int32_t b = (int32_t)(slot / spr);
  const int32_t k = (int32_t)(slot - (uint32_t)b * spr);
  int64_t dbase;
  int32_t gb;
  float T;
  request(P, b, dbase, gb, T);
  if (k > gb) return;
  if (k < gb && blockIdx.x == 0 && tid == 0) {
    put_u32<true>(&P.rec[slot].tok, (uint32_t)P.tokens[dbase + k]);
    put_u32<true>(&P.rec[slot].u, 0u);
  }
  const int64_t lo = (int64_t)blockIdx.x * P.split_len;
  const int64_t hi = lo + P.split_len < P.V ? lo + P.split_len : P.V;
  const Store *tile =
      static_cast<const Store *>(row_ptr<DT>(P.target, dbase + b + k, P.V)) + lo / W;
  const int32_t nu = (int32_t)((hi - lo + W - 1) / W);
  typename U::Raw raw[NV];
  load_tile<DT, VEC, NV>(tile, nu, raw);
  tile_stats<DT, VEC, NV, true>(raw, tile, nu, lo, hi, 0.f, -1,
                                P.parts + (int64_t)slot * P.nsplit + blockIdx.x, &P.rec[slot].z,
                                sh);
  wait_memory();
  __syncthreads();
  const uint32_t n = (uint32_t)(gb + 1) * (uint32_t)P.nsplit;  // tiles of the request
  if (tid == 0)
    s_last = __hip_atomic_fetch_add(&P.arrive[b * kCounterStride], 1u, __ATOMIC_RELAXED,
                                    __HIP_MEMORY_SCOPE_AGENT) == n - 1u;
  __syncthreads();
  if (!s_last) return;
  if (tid == 0)
    __hip_atomic_store(&P.arrive[b * kCounterStride], 0u, __ATOMIC_RELAXED,
                       __HIP_MEMORY_SCOPE_AGENT);
  int64_t db;
  int32_t g;
  bool smp;
  finish_head<kRsThreads, true>(P, b, true, L, db, g, smp);
}

// ------------------------------------------------------------------ k_onepass

// A request's one-launch counters back to zero: the 64-bit arrival word and the completed
// spans.
__device__ __forceinline__ void reset_request_counters(unsigned long long *word, uint32_t *done) {
  __hip_atomic_store(word, 0ull, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  __hip_atomic_store(done, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// The whole step in one launch, for small calls.  Workgroups (tile, row slot) as k_rowstats:
// each computes its tile's statistics, hands the partial over with device-scope atomic stores,
// waits for them to complete and counts itself in on its request's 64-bit arrival word (low
// half: arrivals; high half: spans handed over), whose old value gives its arrival rank.
//  - A greedy request (T = 0) is finished by its last arrival: merge and comparisons, as
//    k_finish's slice 0.  Nothing waits.
//  - A sampled request's stop row(s) are cut into spans of whole 64-unit chunks, at most one
//    per tile and at most 32; the workgroup of arrival rank r owns span r.  An owner that is
//    not the last arrival waits (bounded polling) for the request's last tile, then merges and
//    tests (every workgroup reaches the same decision from the same partials) and sums its
//    span.  The last arrival merges, tests, writes the outputs and sums its own span, if any.
//    A span's chunk sums are published before its completion is counted, and the workgroup
//    whose count completes the last span draws, as k_finish's last slice does.
//  - An owner whose bound runs out (its siblings are not all resident: other work holds the
//    device) hands its span over by adding its bit to the high half of the arrival word.  The
//    last arrival's own arrival returns the spans handed over before it, and it sums those as
//    well; an owner whose hand-over finds every tile already in has handed nothing (the last
//    arrival read the word before) and goes on.  So the waits decide only who sums a span,
//    never a result, and every span is summed exactly once.
//  - Every other touch of a request's counters (arrivals, polls and hand-overs by owners, each
//    followed by that owner's completion or exit) happens before the count completes, so the
//    drawing workgroup returns the counters to zero before it draws: every call leaves them
//    as it found them.
template <int DT, bool VEC>
__global__ __launch_bounds__(kRsThreads) void k_onepass(Params P) {
  using U = Unit<DT, VEC>;
  using Store = typename U::Store;
  constexpr int W = U::W;
  constexpr int NV = int(kTileElems / kRsThreads) / W;
  static_assert(kThreads == kRsThreads, "the finishing steps run on a k_rowstats workgroup");
  __shared__ StatsLds sh;
  __shared__ ReqLds L;
  __shared__ DrawLds<kWaves> D;
  __shared__ int32_t s_go;
  __shared__ uint32_t s_rank;
  __shared__ uint32_t s_handed;
  const int tid = threadIdx.x;
  const uint32_t slot = blockIdx.y + blockIdx.z * gridDim.y;
  const uint32_t spr = (uint32_t)P.spr;
  if (slot >= (uint32_t)P.B * spr) return;
  const int32_t b = (int32_t)(slot / spr);
  const int32_t k = (int32_t)(slot - (uint32_t)b * spr);
  int64_t dbase;
  int32_t gb;
  float T;
  request(P, b, dbase, gb, T);
  const bool sampling = T > 0.f;
  // the row of slot k: target rows 0..gb (slot k), then draft rows (slot gamma+1+i)
  const void *base;
  int64_t row;
  int32_t pos;
  if (k <= P.gamma) {
    if (k > gb) return;
    base = P.target;
    row = dbase + b + k;
    pos = k;
  } else {
    const int32_t i = k - P.gamma - 1;
    if (i >= gb || !sampling) return;
    base = P.draft;
    row = dbase + i;
    pos = i;
  }
  const int64_t lo = (int64_t)blockIdx.x * P.split_len;
  const int64_t hi = lo + P.split_len < P.V ? lo + P.split_len : P.V;
  const Store *tile = static_cast<const Store *>(row_ptr<DT>(base, row, P.V)) + lo / W;
  const int32_t nu = (int32_t)((hi - lo + W - 1) / W);
  {
    // the tile's loads go out first: the token and its record wait on their own round trip
    typename U::Raw raw[NV];
    load_tile<DT, VEC, NV>(tile, nu, raw);
    const int32_t xtok = pos < gb ? P.tokens[dbase + pos] : -1;
    if (k <= P.gamma && pos < gb && blockIdx.x == 0 && tid == 0) {
      put_u32<true>(&P.rec[slot].tok, (uint32_t)xtok);
      put_u32<true>(&P.rec[slot].u,
                    __float_as_uint(sampling ? P.uniforms[2 * (dbase + b + pos)] : 0.f));
    }
    tile_stats<DT, VEC, NV, true>(raw, tile, nu, lo, hi, T, sampling ? xtok : -1,
                                  P.parts + (int64_t)slot * P.nsplit + blockIdx.x,
                                  &P.rec[slot].z, sh);
  }

  // Arrival: this workgroup's stores are complete before it counts itself in.
  const int32_t nrows = gb + 1 + (sampling ? gb : 0);
  const uint32_t n = (uint32_t)nrows * (uint32_t)P.nsplit;  // the request's tiles
  // Spans of whole 64-unit chunks, at most one per tile and at most 32.
  const int64_t nunits = (P.V + W - 1) / W;
  const int64_t most = n < 32u ? (int64_t)n : 32;
  const int64_t su = ceil_div_dev(ceil_div_dev(nunits, most), kChunkUnits) * kChunkUnits;
  const uint32_t nspans = (uint32_t)ceil_div_dev(nunits, su);
  wait_memory();
  __syncthreads();
  // Request b's arrival word (its 128-byte line of `arrive`) and completed spans (its line of
  // `odone`).
  unsigned long long *word =
      reinterpret_cast<unsigned long long *>(&P.arrive[b * kCounterStride]);
  uint32_t *done = &P.odone[b * kCounterStride];
  if (tid == 0) {
    const unsigned long long was =
        __hip_atomic_fetch_add(word, 1ull, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    const uint32_t rank = (uint32_t)was;
    int32_t go;  // 2: the last arrival; 1: an owner that goes on; 0: nothing (more) to do
    if (rank == n - 1u) {
      go = 2;
    } else if (!sampling || rank >= nspans) {
      go = 0;
    } else {
      go = 1;
      uint32_t spins = 0;
      while ((uint32_t)__hip_atomic_load(word, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) < n) {
        __builtin_amdgcn_s_sleep(1);
        if (++spins == P.spin_limit) {  // hand the span over, unless the last tile is in
          const unsigned long long now = __hip_atomic_fetch_add(
              word, 1ull << (32 + rank), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
          go = (uint32_t)now == n ? 1 : 0;
          break;
        }
      }
    }
    s_go = go;
    s_rank = rank;
    s_handed = go == 2 ? (uint32_t)(was >> 32) : 0u;
  }
  __syncthreads();
  const int32_t go = s_go;
  if (go == 0) return;
  int64_t db;
  int32_t g;
  bool smp;
  if (!sampling) {  // a greedy request: its last arrival finishes it
    if (tid == 0) __hip_atomic_store(word, 0ull, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    finish_head<kThreads, true>(P, b, true, L, db, g, smp);
    return;
  }
  const TempConst tc = finish_head<kThreads, true>(P, b, go == 2, L, db, g, smp);
  const Stop st = make_stop(L, gb, P.gamma + 1, tc, dbase + b + L.j, dbase + L.j);
  double *cs = P.chunk_sums + (int64_t)b * P.chunk_stride;
  uint32_t mine = s_handed;  // spans this workgroup sums: its own, and those handed over
  if (s_rank < nspans) mine |= 1u << s_rank;
  if (mine == 0) return;     // the last arrival without a span: the outputs were its part
  const uint32_t count = (uint32_t)__popc(mine);
  while (mine) {
    const int32_t c = __ffs((int)mine) - 1;
    mine &= mine - 1u;
    const int64_t ub = (int64_t)c * su;
    const int64_t ue = ub + su < nunits ? ub + su : nunits;
    stream_chunks<DT, VEC, kThreads, kFinRU>(P, st, ub, ue, cs);
  }
  wait_memory();
  __syncthreads();
  if (tid == 0) {
    const uint32_t before =
        __hip_atomic_fetch_add(done, count, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    s_go = before + count == nspans;
    if (s_go) reset_request_counters(word, done);
  }
  __syncthreads();
  if (s_go) draw_token<DT, VEC, kThreads>(P, b, st, cs, D);  // every span's chunk sums are in
}

// ------------------------------------------------------------------ k_commit

struct CommitParams {
  const int32_t *out_tokens, *out_n, *cu;
  int32_t B, gamma;
  int32_t *seq;
  int64_t capacity;
  int32_t *seq_len;
  unsigned long long *stats, *hist;
};

// One thread per request: append the request's n_b + 1 emitted tokens to its history at
// seq_len[b], clamp the length at capacity, and fold the step into the counters (wavefront
// sums and an LDS histogram, then one device atomic per counter and bin per workgroup).  A
// count outside the verification's range is device data the host cannot check: a negative one
// leaves the request alone and uncounted, one above gamma_b is clamped (memory safety only).
__global__ __launch_bounds__(kThreads) void k_commit(CommitParams C) {
  __shared__ unsigned long long s_sum[5][kWaves];
  __shared__ uint32_t s_hist[SPEC_MAX_GAMMA + 1];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  if (C.hist)
    for (int i = tid; i <= C.gamma; i += kThreads) s_hist[i] = 0u;
  __syncthreads();
  const int64_t b = (int64_t)blockIdx.x * kThreads + tid;
  unsigned long long v[5] = {0, 0, 0, 0, 0};
  if (b < C.B && C.out_n[b] >= 0) {
    int64_t dbase, gb;
    if (C.cu) {
      dbase = C.cu[b];
      gb = (int64_t)C.cu[b + 1] - dbase;
    } else {
      dbase = b * C.gamma;
      gb = C.gamma;
    }
    // memory safety on device data the host cannot check
    gb = gb < 0 ? 0 : (gb > C.gamma ? C.gamma : gb);
    int64_t n = C.out_n[b];
    n = n > gb ? gb : n;
    int64_t len = C.seq_len[b];
    len = len < 0 ? 0 : (len > C.capacity ? C.capacity : len);
    const int32_t *src = C.out_tokens + dbase + b;
    int32_t *dst = C.seq + b * C.capacity;
    for (int64_t i = 0; i <= n; ++i)
      if (len + i < C.capacity) dst[len + i] = src[i];
    const int64_t end = len + n + 1;
    C.seq_len[b] = (int32_t)(end < C.capacity ? end : C.capacity);
    v[0] = (unsigned long long)gb;
    v[1] = (unsigned long long)n;
    v[2] = (unsigned long long)(n + 1);
    v[3] = 1ull;
    v[4] = (unsigned long long)(end > C.capacity ? end - C.capacity : 0);
    if (C.hist) atomicAdd(&s_hist[n], 1u);
  }
  if (C.stats) {
#pragma unroll
    for (int k = 0; k < 5; ++k) {
      unsigned long long x = v[k];
      for (int o = 32; o > 0; o >>= 1) x += __shfl_xor(x, o);
      if (lane == 0) s_sum[k][wave] = x;
    }
  }
  __syncthreads();
  if (C.stats && tid < 5) {
    unsigned long long x = 0;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) x += s_sum[tid][w];
    if (x) atomicAdd(&C.stats[tid], x);
  }
  if (C.hist)
    for (int i = tid; i <= C.gamma; i += kThreads)
      if (s_hist[i]) atomicAdd(&C.hist[i], (unsigned long long)s_hist[i]);
}

// ------------------------------------------------------------------ n-gram drafter

constexpr int kNgramThreads = 512;  // a request's workgroup: contexts of up to 8192 tokens
                                    // take one round (measured 20-25% faster than 256)
constexpr int kNgramLoads = 16;     // context tokens per thread in flight
constexpr int kNgramWaves = kNgramThreads / 64;

struct NgramParams {
  const int32_t *seq;
  int64_t capacity;
  const int32_t *seq_len;
  int32_t B, n_min, n_max, gamma;
  int32_t *counts, *dense, *cu, *packed;
};

// One workgroup per request.  With h the context and L its length, m(e) is the length of the
// common run of h ending at e and h ending at L - 1 (compared backwards, capped at
// n_hi = min(n_max, L - 1)), for every e < L - 1: an n-gram equal to the last n tokens ends
// at e iff m(e) >= n.  So the longest usable n is the maximum of m, and its earliest
// occurrence ends at the first e attaining it; one pass over the context and one block
// reduction of the key (m, -e) give both.  The context goes through LDS a round of
// kNgramRound tokens at a time, behind a halo of the previous round's last SPEC_NGRAM_MAX_N
// tokens, so the backward comparisons read LDS; the first round's loads go out with the
// pattern's, and each next round's while the current one is compared.
constexpr int kNgramRound = kNgramThreads * kNgramLoads;
__global__ __launch_bounds__(kNgramThreads) void k_ngram(NgramParams G) {
  __shared__ int32_t s_suf[SPEC_NGRAM_MAX_N];  // s_suf[k] = h[L - 1 - k]
  __shared__ int32_t s_ctx[SPEC_NGRAM_MAX_N + kNgramRound];  // halo, then the round
  __shared__ unsigned long long s_key[kNgramWaves];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int64_t b = blockIdx.x;
  const int32_t *h = G.seq + b * G.capacity;
  int64_t L = G.seq_len[b];
  L = L < 0 ? 0 : (L > G.capacity ? G.capacity : L);
  const int32_t n_hi = (int32_t)(L - 1 < G.n_max ? L - 1 : G.n_max);
  int32_t cnt = 0;
  int64_t start = 0;
  if (n_hi >= G.n_min) {  // uniform across the workgroup
    const int64_t E = L - 1;  // candidate ends e < E
    int32_t v[kNgramLoads];
#pragma unroll
    for (int q = 0; q < kNgramLoads; ++q) {
      const int64_t e = q * kNgramThreads + tid;
      v[q] = e < E ? h[e] : 0;
    }
    if (tid < n_hi) s_suf[tid] = h[L - 1 - tid];
    // key = m << 32 | (2^31 - 1 - e): the maximum has the largest m and, for it, the
    // smallest e.
    unsigned long long key = 0;
    for (int64_t e0 = 0; e0 < E; e0 += kNgramRound) {
#pragma unroll
      for (int q = 0; q < kNgramLoads; ++q) s_ctx[SPEC_NGRAM_MAX_N + q * kNgramThreads + tid] = v[q];
      __syncthreads();
      const int32_t last = s_suf[0];
      int32_t cur[kNgramLoads];
#pragma unroll
      for (int q = 0; q < kNgramLoads; ++q) cur[q] = v[q];
      const int64_t e1 = e0 + kNgramRound;
      if (e1 < E) {  // the next round's loads go out before this round is compared
#pragma unroll
        for (int q = 0; q < kNgramLoads; ++q) {
          const int64_t e = e1 + q * kNgramThreads + tid;
          v[q] = e < E ? h[e] : 0;
        }
      }
#pragma unroll
      for (int q = 0; q < kNgramLoads; ++q) {
        const int64_t e = e0 + q * kNgramThreads + tid;
        if (e < E && cur[q] == last) {
          const int32_t at = SPEC_NGRAM_MAX_N + q * kNgramThreads + tid;  // e's slot in s_ctx
          int32_t k = 1;
          while (k < n_hi && e - k >= 0 && s_ctx[at - k] == s_suf[k]) ++k;
          const unsigned long long kk =
              ((unsigned long long)k << 32) | (unsigned long long)(0x7fffffffll - e);
          key = kk > key ? kk : key;
        }
      }
      __syncthreads();  // every comparison of this round is done
      if (e1 < E) {     // uniform: this round was full, its tail becomes the next halo
        int32_t t = 0;
        if (tid < SPEC_NGRAM_MAX_N) t = s_ctx[kNgramRound + tid];
        __syncthreads();  // the tail is read before the next round overwrites it
        if (tid < SPEC_NGRAM_MAX_N) s_ctx[tid] = t;
      }
    }
    for (int o = 32; o > 0; o >>= 1) {
      const unsigned long long t = __shfl_xor(key, o);
      key = t > key ? t : key;
    }
    if (lane == 0) s_key[wave] = key;
    __syncthreads();
#pragma unroll
    for (int w = 0; w < kNgramWaves; ++w) key = s_key[w] > key ? s_key[w] : key;
    const int32_t n = (int32_t)(key >> 32);
    if (n >= G.n_min) {
      const int64_t e = 0x7fffffffll - (int64_t)(key & 0xffffffffull);
      start = e + 1;  // the token after the occurrence (j + n with j = e - n + 1)
      cnt = (int32_t)(L - start < G.gamma ? L - start : G.gamma);
    }
  }
  for (int i = tid; i < G.gamma; i += kNgramThreads)
    G.dense[b * G.gamma + i] = i < cnt ? h[start + i] : -1;
  if (tid == 0) G.counts[b] = cnt;
}

// One workgroup: running exclusive scan of the counts into cu (the verification step's CSR
// over draft rows) and the proposals packed behind it, kNgramPackThreads requests at a time.
constexpr int kNgramPackThreads = 1024;
__global__ __launch_bounds__(kNgramPackThreads) void k_ngram_pack(NgramParams G) {
  constexpr int NW = kNgramPackThreads / 64;
  __shared__ int32_t s_tot[NW];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  int64_t base = 0;
  for (int64_t b0 = 0; b0 < G.B; b0 += kNgramPackThreads) {
    const int64_t b = b0 + tid;
    const int32_t c = b < G.B ? G.counts[b] : 0;
    int32_t inc = c;
    for (int o = 1; o < 64; o <<= 1) {
      const int32_t t = __shfl_up(inc, o);
      if (lane >= o) inc += t;
    }
    if (lane == 63) s_tot[wave] = inc;
    __syncthreads();
    int32_t off = 0, total = 0;
#pragma unroll
    for (int w = 0; w < NW; ++w) {
      if (w < wave) off += s_tot[w];
      total += s_tot[w];
    }
    __syncthreads();
    const int64_t first = base + off + inc - c;
    if (b < G.B) {
      G.cu[b] = (int32_t)first;
      for (int32_t i = 0; i < c; ++i) G.packed[first + i] = G.dense[b * G.gamma + i];
    }
    base += total;
  }
  if (tid == 0) G.cu[G.B] = (int32_t)base;
}

// ------------------------------------------------------------------ host side

struct Plan {
  int32_t spr, nsplit;       // row slots per request; k_rowstats tiles per row
  int64_t split_len, chunk_stride;
  size_t off_sync, off_parts, off_rec, off_chunks, off_done, total;
};

size_t align_up(size_t x) { return (x + kAlign - 1) / kAlign * kAlign; }
int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }

bool make_plan(int32_t B, int32_t gamma, int64_t V, int dtype, bool greedy, Plan &pl) {
  if (B < 0 || gamma < 0 || gamma > SPEC_MAX_GAMMA || V < 1 || V > kMaxV) return false;
  if (dtype != SPEC_F32 && dtype != SPEC_BF16) return false;
  const int64_t bb = B > 0 ? B : 1;
  pl.spr = greedy ? gamma + 1 : 2 * gamma + 1;
  const int64_t rows = bb * (gamma + 1 + (greedy ? 0 : gamma));
  // k_rowstats: one tile per workgroup; small problems get finer (partial) tiles.
  const int64_t tiles = ceil_div(V, kTileElems);
  const int64_t ns = tiles;
  int64_t len = kTileElems;
  if (tiles * rows < kSmallGrid && tiles < kMaxSlices) {
    int64_t want = ceil_div(kSmallGrid, rows);
    const int64_t cap = ceil_div(V, 2048);
    if (want > cap) want = cap;
    if (want > kMaxSlices) want = kMaxSlices;
    if (want > ns) len = ceil_div(ceil_div(V, want), 8) * 8;
  }
  pl.nsplit = (int32_t)ceil_div(V, len);  // no empty slice
  pl.split_len = len;
  // (k_onepass uses whole kTileElems tiles: never more per row than k_rowstats)
  // Chunk sums of the stop rows; the element path (one element per unit) has the most chunks.
  pl.chunk_stride = ceil_div(V, kChunkUnits);
  // The one-launch counters sit first, at the same place and size for every call, so that
  // calls of any shape find them as the last call left them: zero.
  pl.off_sync = 0;
  pl.off_parts = align_up(2 * (size_t)kOneMaxB * kCounterStride * sizeof(uint32_t));
  pl.off_rec = pl.off_parts + align_up((size_t)bb * pl.spr * pl.nsplit * sizeof(Partial));
  pl.off_chunks = pl.off_rec + align_up((size_t)bb * pl.spr * sizeof(SlotRec));
  pl.off_done = pl.off_chunks +
                (greedy ? 0 : align_up((size_t)bb * pl.chunk_stride * sizeof(double)));
  pl.total = pl.off_done + align_up((size_t)bb * kCounterStride * sizeof(uint32_t));
  return true;
}

#define SPEC_TRY(expr)              \
  do {                              \
    const int rc_ = (expr);         \
    if (rc_ != SPEC_OK) return rc_; \
  } while (0)

// Launch kernel k of the call.  With probe events for it, the dispatch itself records them
// (hipExtLaunchKernel), so timing adds no marker packets, and no idle time, to the stream.
template <typename K>
int launch(K kernel, dim3 grid, int threads, const spec_probe *probe, int k, hipStream_t s,
           Params &P) {
  hipEvent_t e0 = probe ? static_cast<hipEvent_t>(probe->events[2 * k]) : nullptr;
  hipEvent_t e1 = probe ? static_cast<hipEvent_t>(probe->events[2 * k + 1]) : nullptr;
  if (!e0 && !e1) {
    kernel<<<grid, dim3(threads), 0, s>>>(P);
    return hipGetLastError() == hipSuccess ? SPEC_OK : SPEC_ERR_HIP;
  }
  void *args[] = {&P};
  return hipExtLaunchKernel(reinterpret_cast<const void *>(kernel), grid, dim3(threads), args, 0,
                            s, e0, e1, 0) == hipSuccess
             ? SPEC_OK
             : SPEC_ERR_HIP;
}

// Workgroups of `kernel` (kThreads each) the current device holds at once; 0 if unknown.
int resident_capacity(const void *kernel) {
  int dev = 0, cus = 0, per = 0;
  if (hipGetDevice(&dev) != hipSuccess ||
      hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
      hipOccupancyMaxActiveBlocksPerMultiprocessor(&per, kernel, kThreads, 0) != hipSuccess) {
    (void)hipGetLastError();  // leave no error behind for the launch check
    return 0;
  }
  return per * cus;
}

// The library's own choice of one launch, where it measured faster on MI355X: calls of at most
// kOneAutoTiles row tiles with 16-byte aligned rows (and, with sampled requests, within three
// quarters of the device's resident capacity).  Larger calls measured faster or equal in two
// launches (greedy: 4608 tiles equal, 41472 tiles 25% slower in one).
constexpr int64_t kOneAutoTiles = 2048;

template <int DT, bool VEC>
int run(Params P, const Plan &pl, const spec_probe *probe, hipStream_t s) {
  const int asked = probe ? probe->path : SPEC_PATH_AUTO;
  P.spin_limit = probe && probe->spin_limit ? probe->spin_limit : kSpinLimit;
  if (asked != SPEC_PATH_AUTO && asked != SPEC_PATH_TWO && asked != SPEC_PATH_ONE)
    return SPEC_ERR_SHAPE;
  const int64_t slots = (int64_t)P.B * pl.spr;
  const uint32_t gy = (uint32_t)(slots < kMaxGridY ? slots : kMaxGridY);
  const uint32_t gz = (uint32_t)ceil_div(slots, gy);
  if (asked != SPEC_PATH_TWO && P.B <= kOneMaxB) {
    // one launch: whole kTileElems tiles; a call with sampled requests also needs all of its
    // workgroups resident at once (three quarters of the device's capacity, to spare)
    const int64_t ns = ceil_div(P.V, kTileElems);
    const int64_t tiles = slots * ns;
    bool one = asked == SPEC_PATH_ONE || (VEC && tiles <= kOneAutoTiles);
    if (one && !P.greedy_all)
      one = tiles * 4 <= 3 * (int64_t)resident_capacity(
                                 reinterpret_cast<const void *>(k_onepass<DT, VEC>));
    if (one) {
      P.nsplit = (int32_t)ns;
      P.split_len = kTileElems;
      const dim3 grid((uint32_t)ns, gy, gz);
      // greedy calls: k_greedy1, whose greedy-only code measured faster than k_onepass's
      return P.greedy_all ? launch(k_greedy1<DT, VEC>, grid, kRsThreads, probe, 0, s, P)
                          : launch(k_onepass<DT, VEC>, grid, kRsThreads, probe, 0, s, P);
    }
  }
  if (asked == SPEC_PATH_ONE) return SPEC_ERR_SHAPE;
  // k_finish: enough slices of the stop rows per request for about kFinGrid workgroups, each
  // at least one pass and a whole number of 64-unit chunks.  Greedy calls need slice 0 only.
  const int64_t nunits = ceil_div(P.V, Unit<DT, VEC>::W);
  int64_t want = P.greedy_all ? 1 : ceil_div(kFinGrid, P.B);
  const int64_t most = ceil_div(nunits, kFinPassUnits);
  if (want > most) want = most;
  P.slice_units = ceil_div(ceil_div(nunits, want), kChunkUnits) * kChunkUnits;
  P.nslice = (int32_t)ceil_div(nunits, P.slice_units);
  const int64_t groups = ceil_div(P.B, 8);  // k_finish: requests in groups of eight, one per XCD
  const uint32_t fy = (uint32_t)(groups < kMaxGridY ? groups : kMaxGridY);
  const uint32_t fz = (uint32_t)ceil_div(groups, fy);
  SPEC_TRY(launch(k_rowstats<DT, VEC>, dim3((uint32_t)pl.nsplit, gy, gz), kRsThreads, probe, 0,
                  s, P));
  SPEC_TRY(launch(k_finish<DT, VEC>, dim3((uint32_t)P.nslice * 8u, fy, fz), kThreads, probe, 1, s,
                  P));
  return SPEC_OK;
}

bool aligned16(const void *p) { return ((uintptr_t)p & 15u) == 0; }

int check_shape(int32_t B, int32_t gamma, int64_t V, int dtype) {
  if (dtype != SPEC_F32 && dtype != SPEC_BF16) return SPEC_ERR_DTYPE;
  if (B < 0 || gamma < 0 || gamma > SPEC_MAX_GAMMA || V < 1 || V > kMaxV) return SPEC_ERR_SHAPE;
  return SPEC_OK;
}

int setup(Params &P, const Plan &pl, void *workspace, size_t workspace_bytes) {
  if (!workspace) return SPEC_ERR_NULL;
  if (((uintptr_t)workspace & (kAlign - 1)) != 0 || workspace_bytes < pl.total)
    return SPEC_ERR_WORKSPACE;
  if ((int64_t)P.B * pl.spr > kMaxGridY * kMaxGridY) return SPEC_ERR_SHAPE;
  char *ws = static_cast<char *>(workspace);
  P.parts = reinterpret_cast<Partial *>(ws + pl.off_parts);
  P.rec = reinterpret_cast<SlotRec *>(ws + pl.off_rec);
  P.done = reinterpret_cast<uint32_t *>(ws + pl.off_done);
  P.arrive = reinterpret_cast<uint32_t *>(ws + pl.off_sync);
  P.odone = P.arrive + (size_t)kOneMaxB * kCounterStride;
  P.chunk_sums = reinterpret_cast<double *>(ws + pl.off_chunks);
  P.chunk_stride = pl.chunk_stride;
  P.spr = pl.spr;
  P.nsplit = pl.nsplit;
  P.split_len = pl.split_len;
  return SPEC_OK;
}

template <int DT>
int dispatch(const Params &P, const Plan &pl, const spec_probe *probe, hipStream_t s, bool vec) {
  return vec ? run<DT, true>(P, pl, probe, s) : run<DT, false>(P, pl, probe, s);
}

// ------------------------------------------------------------------ the static scratch

// The allocation-free entry point's workspace: one array per device, in the code object's
// zero-initialised device data, kept until the process ends.  Zero at load, which is what the
// one-launch counters at its start need, and every call returns them to zero.  Host code never
// passes `scratch` itself (on the host its name is a stand-in, not a device address): it uses
// the address hipGetSymbolAddress gives for the current device, fetched once per device.
static __device__ __align__(256) unsigned char scratch[SPEC_STATIC_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;
std::atomic<void *> g_scratch_addr[kMaxDevices];

// The current device's address of `scratch` (nullptr if it cannot be had).
void *scratch_address() {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) {
    (void)hipGetLastError();
    return nullptr;
  }
  void *ptr = g_scratch_addr[dev].load(std::memory_order_acquire);
  if (ptr) return ptr;
  if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)) != hipSuccess || !ptr) {
    (void)hipGetLastError();
    return nullptr;
  }
  g_scratch_addr[dev].store(ptr, std::memory_order_release);  // the same value for any racer
  return ptr;
}

}  // namespace

extern "C" {

size_t spec_verify_workspace_size(int32_t B, int32_t gamma, int64_t V, int dtype) {
  Plan a, b;
  if (!make_plan(B, gamma, V, dtype, false, a) || !make_plan(B, gamma, V, dtype, true, b))
    return 0;
  return a.total > b.total ? a.total : b.total;
}

const char *spec_verify_strerror(int code) {
  switch (code) {
    case SPEC_OK: return "success";
    case SPEC_ERR_NULL: return "a required pointer is NULL";
    case SPEC_ERR_SHAPE:
      return "invalid sizes (B < 0, gamma outside [0, 64], V outside [1, 2^24], or grid too large)";
    case SPEC_ERR_DTYPE: return "dtype is neither SPEC_F32 nor SPEC_BF16";
    case SPEC_ERR_WORKSPACE: return "workspace too small or not 256-byte aligned";
    case SPEC_ERR_HIP: return "HIP kernel launch failed";
    case SPEC_ERR_TOO_LARGE:
      return "the call needs more scratch than the static buffer holds "
             "(SPEC_STATIC_SCRATCH_BYTES; spec_verify_workspace_size gives the need)";
    default: return "unknown spec_verify error code";
  }
}

int spec_verify_sample(const void *target_logits, const void *draft_logits, int dtype,
                       const int32_t *draft_tokens, const float *uniforms,
                       const float *temperatures, int32_t B, int32_t gamma,
                       const int32_t *cu_draft, int64_t V, int32_t *out_tokens,
                       int32_t *out_num_accepted, void *workspace, size_t workspace_bytes,
                       const spec_probe *probe, void *stream) {
  SPEC_TRY(check_shape(B, gamma, V, dtype));
  if (B == 0) return SPEC_OK;
  if (!target_logits || !draft_logits || !draft_tokens || !uniforms || !temperatures ||
      !out_tokens || !out_num_accepted)
    return SPEC_ERR_NULL;
  Plan pl;
  if (!make_plan(B, gamma, V, dtype, false, pl)) return SPEC_ERR_SHAPE;
  Params P = {};
  P.target = target_logits;
  P.draft = draft_logits;
  P.tokens = draft_tokens;
  P.uniforms = uniforms;
  P.temps = temperatures;
  P.cu = cu_draft;
  P.B = B;
  P.gamma = gamma;
  P.V = V;
  P.out_tokens = out_tokens;
  P.out_n = out_num_accepted;
  P.greedy_all = 0;
  SPEC_TRY(setup(P, pl, workspace, workspace_bytes));
  if (probe) {
    P.p_x = probe->p_x;
    P.q_x = probe->q_x;
    P.row_max_t = probe->row_max_t;
    P.row_sum_t = probe->row_sum_t;
    P.row_max_d = probe->row_max_d;
    P.row_sum_d = probe->row_sum_d;
    P.resid_mass = probe->resid_mass;
  }
  const int es = dtype == SPEC_F32 ? 4 : 2;
  const bool vec = aligned16(target_logits) && aligned16(draft_logits) && (V * es) % 16 == 0;
  hipStream_t s = static_cast<hipStream_t>(stream);
  return dtype == SPEC_F32 ? dispatch<SPEC_F32>(P, pl, probe, s, vec)
                           : dispatch<SPEC_BF16>(P, pl, probe, s, vec);
}

int spec_verify_sample_static(const void *target_logits, const void *draft_logits, int dtype,
                              const int32_t *draft_tokens, const float *uniforms,
                              const float *temperatures, int32_t B, int32_t gamma,
                              const int32_t *cu_draft, int64_t V, int32_t *out_tokens,
                              int32_t *out_num_accepted, const spec_probe *probe,
                              void *stream) {
  SPEC_TRY(check_shape(B, gamma, V, dtype));
  if (B == 0) return SPEC_OK;
  if (!target_logits || !draft_logits || !draft_tokens || !uniforms || !temperatures ||
      !out_tokens || !out_num_accepted)
    return SPEC_ERR_NULL;
  const size_t need = spec_verify_workspace_size(B, gamma, V, dtype);
  if (need == 0) return SPEC_ERR_SHAPE;
  if (need > SPEC_STATIC_SCRATCH_BYTES) return SPEC_ERR_TOO_LARGE;
  void *ws = scratch_address();
  if (!ws) return SPEC_ERR_HIP;
  return spec_verify_sample(target_logits, draft_logits, dtype, draft_tokens, uniforms,
                            temperatures, B, gamma, cu_draft, V, out_tokens, out_num_accepted, ws,
                            SPEC_STATIC_SCRATCH_BYTES, probe, stream);
}

int spec_verify_greedy(const void *target_logits, int dtype, const int32_t *draft_tokens,
                       int32_t B, int32_t gamma, const int32_t *cu_draft, int64_t V,
                       int32_t *out_tokens, int32_t *out_num_accepted, void *workspace,
                       size_t workspace_bytes, const spec_probe *probe, void *stream) {
  SPEC_TRY(check_shape(B, gamma, V, dtype));
  if (B == 0) return SPEC_OK;
  if (!target_logits || !draft_tokens || !out_tokens || !out_num_accepted) return SPEC_ERR_NULL;
  Plan pl;
  if (!make_plan(B, gamma, V, dtype, true, pl)) return SPEC_ERR_SHAPE;
  Params P = {};
  P.target = target_logits;
  P.draft = nullptr;
  P.tokens = draft_tokens;
  P.cu = cu_draft;
  P.B = B;
  P.gamma = gamma;
  P.V = V;
  P.out_tokens = out_tokens;
  P.out_n = out_num_accepted;
  P.greedy_all = 1;
  SPEC_TRY(setup(P, pl, workspace, workspace_bytes));
  if (probe) P.row_max_t = probe->row_max_t;
  const int es = dtype == SPEC_F32 ? 4 : 2;
  const bool vec = aligned16(target_logits) && (V * es) % 16 == 0;
  hipStream_t s = static_cast<hipStream_t>(stream);
  return dtype == SPEC_F32 ? dispatch<SPEC_F32>(P, pl, probe, s, vec)
                           : dispatch<SPEC_BF16>(P, pl, probe, s, vec);
}

int spec_verify_commit(const int32_t *out_tokens, const int32_t *out_num_accepted,
                       const int32_t *cu_draft, int32_t B, int32_t gamma, int32_t *seq_tokens,
                       int64_t capacity, int32_t *seq_len, uint64_t *stats,
                       uint64_t *accept_hist, void *stream) {
  if (B < 0 || gamma < 0 || gamma > SPEC_MAX_GAMMA || capacity < 0) return SPEC_ERR_SHAPE;
  if (B == 0) return SPEC_OK;
  if (!out_tokens || !out_num_accepted || !seq_tokens || !seq_len) return SPEC_ERR_NULL;
  if ((int64_t)B > (int64_t)INT32_MAX - kThreads) return SPEC_ERR_SHAPE;
  CommitParams C = {};
  C.out_tokens = out_tokens;
  C.out_n = out_num_accepted;
  C.cu = cu_draft;
  C.B = B;
  C.gamma = gamma;
  C.seq = seq_tokens;
  C.capacity = capacity;
  C.seq_len = seq_len;
  C.stats = reinterpret_cast<unsigned long long *>(stats);
  C.hist = reinterpret_cast<unsigned long long *>(accept_hist);
  k_commit<<<dim3((uint32_t)ceil_div(B, kThreads)), dim3(kThreads), 0,
             static_cast<hipStream_t>(stream)>>>(C);
  return hipGetLastError() == hipSuccess ? SPEC_OK : SPEC_ERR_HIP;
}

int spec_ngram_propose(const int32_t *seq_tokens, int64_t capacity, const int32_t *seq_len,
                       int32_t B, int32_t n_min, int32_t n_max, int32_t gamma,
                       int32_t *out_counts, int32_t *out_dense, int32_t *out_cu,
                       int32_t *out_packed, void *stream) {
  if (B < 0 || capacity < 0 || n_min < 1 || n_max < n_min || n_max > SPEC_NGRAM_MAX_N ||
      gamma < 0 || gamma > SPEC_MAX_GAMMA || capacity > (int64_t)INT32_MAX ||
      (int64_t)B * gamma > (int64_t)INT32_MAX)
    return SPEC_ERR_SHAPE;
  if (B == 0) return SPEC_OK;
  // with gamma == 0 nothing is written to out_dense or out_packed: they may be NULL
  if (!seq_tokens || !seq_len || !out_counts || (gamma > 0 && !out_dense) ||
      (gamma > 0 && (!out_cu) != (!out_packed)))
    return SPEC_ERR_NULL;
  NgramParams G = {};
  G.seq = seq_tokens;
  G.capacity = capacity;
  G.seq_len = seq_len;
  G.B = B;
  G.n_min = n_min;
  G.n_max = n_max;
  G.gamma = gamma;
  G.counts = out_counts;
  G.dense = out_dense;
  G.cu = out_cu;
  G.packed = out_packed;
  hipStream_t s = static_cast<hipStream_t>(stream);
  k_ngram<<<dim3((uint32_t)B), dim3(kNgramThreads), 0, s>>>(G);
  if (hipGetLastError() != hipSuccess) return SPEC_ERR_HIP;
  if (out_cu) {
    k_ngram_pack<<<dim3(1), dim3(kNgramPackThreads), 0, s>>>(G);
    if (hipGetLastError() != hipSuccess) return SPEC_ERR_HIP;
  }
  return SPEC_OK;
}

}  // extern "C"
