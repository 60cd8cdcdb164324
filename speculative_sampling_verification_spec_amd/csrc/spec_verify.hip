// Speculative-sampling verification step for MI355X (CDNA4, gfx950): HIP kernels + C ABI.
//
// The step (pages cited in include/spec_verify.h by title and section): per request, accept
// draft x_i with probability min(1, p_i(x_i)/q_i(x_i)), stop at the first rejection j,
// and emit a draw from max(p_j - q_j, 0) there, or from p_gamma when nothing was rejected;
// at temperature zero, compare each draft with the target argmax instead.
//
// Four launches on the caller's stream, none of which waits for the host:
//   1. k_rowstats  — the HBM-bound stream over every needed logit row, split along V.  Each
//                    workgroup reads one V-slice of one row with 16-byte loads and reduces
//                    it to (max, sum_k 2^((z_k - max) c)) with c = log2(e)/T (online max,
//                    fp32 terms, fp64 sums), or to (max, lowest argmax) for greedy rows.
//   2. k_decide    — one wavefront per request: merges the slice partials in fp64, gathers
//                    the two logits at each draft token, runs the accept tests lane-parallel
//                    and finds the first rejection with a ballot + find-first-set.
//   3. k_resid     — re-reads only the stop row(s) of each sampled request and sums the
//                    residual weights max(p - q, 0) (or p for the bonus) per V-slice.
//   4. k_sample    — one workgroup per sampled request: scans the slice sums, then runs a
//                    block prefix scan inside the chosen slice to find the drawn token.
//
// Numerics: every logit is converted exactly to fp32; per-element exponent arguments use
// the exact difference to the running max and a two-float split of c, so the tempered
// softmax is not shifted by rounding c; sums across elements, lanes, waves and slices are
// fp64.  The accept test and p(x), q(x) are evaluated in fp64 from the gathered logits.  The
// residual weight is computed as p_k (1 - 2^delta_k), delta_k = log2(q_k / p_k) formed in
// fp64, with expm1 for the bracket: it keeps its relative accuracy when p_k and q_k almost
// cancel.
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstddef>
#include <cstdint>

#include "spec_verify.h"

namespace {

constexpr int kThreads = 256;            // 4 wavefronts of 64
constexpr int kWaves = kThreads / 64;
constexpr int kUnroll = 8;               // 16-byte load units in flight per thread
constexpr int kMaxSplits = 64;
constexpr int kMinUnitsPerSplit = 64;
constexpr int kTargetWorkgroups = 2048;  // 8 per CU on 256 CUs
constexpr double kLog2e = 1.4426950408889634074;
constexpr double kLn2 = 0.69314718055994530942;
constexpr size_t kAlign = 256;

enum : int32_t { kModeNone = 0, kModeResidual = 1, kModeBonus = 2 };

// Per (row, V-slice) result of k_rowstats.  Sampled rows: m = raw max, s = sum of
// 2^((z - m) c).  Greedy rows: m = raw max, idx = lowest index attaining it.
struct alignas(16) Partial {
  float m;
  int32_t idx;
  double s;
};

// Per request, written by k_decide for k_resid / k_sample.
struct alignas(64) Stop {
  int32_t j;      // stop row = accepted count
  int32_t mode;   // kModeNone (greedy), kModeResidual, kModeBonus
  float mt, md;   // raw maxima of target / draft row j
  double st, sd;  // their normalisers sum 2^((z - m) c)
  double c;       // log2(e) / T as the exact sum c_hi + c_lo
  double k;       // (mt - md) c + log2(st / sd): log2(q_k/p_k) = (zd_k - zt_k) c + k
  float c_hi, c_lo;
  int32_t pad[2];
};
static_assert(sizeof(Stop) == 64, "Stop layout");

struct Params {
  const void *target, *draft;
  const int32_t *tokens;
  const float *uniforms, *temps;
  const int32_t *cu;
  int32_t B, gamma;
  int64_t V;
  int32_t *out_tokens, *out_n;
  Partial *parts;
  Stop *stop;
  double *rsum;
  int32_t spr;          // row slots per request: 2*gamma+1 (sample) or gamma+1 (greedy)
  int32_t nsplit;       // V-slices per row in k_rowstats
  int64_t split_len;    // elements per slice (multiple of the load width)
  int32_t nsplit_r;     // V-slices per stop row in k_resid
  int64_t split_len_r;
  int32_t greedy_all;
  double *p_x, *q_x, *row_sum_t, *row_sum_d, *resid_mass;
  float *row_max_t, *row_max_d;
};

// ------------------------------------------------------------------ request / row helpers

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
  double c;  // c_hi + c_lo exactly
  float c_hi, c_lo;
};

__device__ __forceinline__ TempConst temp_const(float T) {
  double c = kLog2e / (double)T;
  if (c > 1e38) c = 1e38;
  const float hi = (float)c;
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

// One load unit: 16 bytes (4 fp32 / 8 bf16) when rows are 16-byte aligned, else 1 element.
template <int DT, bool VEC>
struct Unit {
  static constexpr int W = VEC ? (DT == SPEC_F32 ? 4 : 8) : 1;
  __device__ static __forceinline__ void load(const void *row, int64_t u, float (&x)[W]) {
    if constexpr (VEC) {
      const uint4 v = static_cast<const uint4 *>(row)[u];
      if constexpr (DT == SPEC_F32) {
        x[0] = __uint_as_float(v.x);
        x[1] = __uint_as_float(v.y);
        x[2] = __uint_as_float(v.z);
        x[3] = __uint_as_float(v.w);
      } else {
        x[0] = __uint_as_float(v.x << 16);
        x[1] = __uint_as_float(v.x & 0xffff0000u);
        x[2] = __uint_as_float(v.y << 16);
        x[3] = __uint_as_float(v.y & 0xffff0000u);
        x[4] = __uint_as_float(v.z << 16);
        x[5] = __uint_as_float(v.z & 0xffff0000u);
        x[6] = __uint_as_float(v.w << 16);
        x[7] = __uint_as_float(v.w & 0xffff0000u);
      }
    } else {
      x[0] = logit_at<DT>(row, u);
    }
  }
};

template <int DT>
__device__ __forceinline__ const void *row_ptr(const void *base, int64_t row, int64_t V) {
  constexpr int64_t es = DT == SPEC_F32 ? 4 : 2;
  return static_cast<const char *>(base) + row * V * es;
}

// 2^((z - m) c) in fp32 with the exact difference and the split constant.
__device__ __forceinline__ float exp_term(float z, float m, float c_hi, float c_lo) {
  const float d = z - m;
  return __builtin_amdgcn_exp2f(fmaf(d, c_hi, d * c_lo));
}

// ------------------------------------------------------------------ block reductions

__device__ __forceinline__ float wave_max(float v) {
  for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o));
  return v;
}
__device__ __forceinline__ double wave_sum(double v) {
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o);
  return v;
}

__device__ float block_max(float v, float *sh) {
  v = wave_max(v);
  const int w = threadIdx.x >> 6;
  if ((threadIdx.x & 63) == 0) sh[w] = v;
  __syncthreads();
  float r = sh[0];
  for (int i = 1; i < kWaves; ++i) r = fmaxf(r, sh[i]);
  __syncthreads();
  return r;
}

__device__ double block_sum(double v, double *sh) {
  v = wave_sum(v);
  const int w = threadIdx.x >> 6;
  if ((threadIdx.x & 63) == 0) sh[w] = v;
  __syncthreads();
  double r = 0.0;
  for (int i = 0; i < kWaves; ++i) r += sh[i];
  __syncthreads();
  return r;
}

// (max value, lowest index) lexicographic reduction.
__device__ __forceinline__ void argmax_merge(float &bv, int32_t &bi, float ov, int32_t oi) {
  if (ov > bv || (ov == bv && oi < bi)) {
    bv = ov;
    bi = oi;
  }
}

__device__ void block_argmax(float &bv, int32_t &bi, float *shv, int32_t *shi) {
  for (int o = 32; o > 0; o >>= 1) {
    const float ov = __shfl_xor(bv, o);
    const int32_t oi = __shfl_xor(bi, o);
    argmax_merge(bv, bi, ov, oi);
  }
  const int w = threadIdx.x >> 6;
  if ((threadIdx.x & 63) == 0) {
    shv[w] = bv;
    shi[w] = bi;
  }
  __syncthreads();
  bv = shv[0];
  bi = shi[0];
  for (int i = 1; i < kWaves; ++i) argmax_merge(bv, bi, shv[i], shi[i]);
  __syncthreads();
}

// Exclusive scan over the block in thread order (fp64); also returns the block total.
__device__ double block_exclusive_scan(double v, double *sh, double &total) {
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  double inc = v;
  for (int o = 1; o < 64; o <<= 1) {
    const double t = __shfl_up(inc, o);
    if (lane >= o) inc += t;
  }
  if (lane == 63) sh[w] = inc;
  __syncthreads();
  double off = 0.0;
  total = 0.0;
  for (int i = 0; i < kWaves; ++i) {
    if (i < w) off += sh[i];
    total += sh[i];
  }
  __syncthreads();
  return off + inc - v;
}

// ------------------------------------------------------------------ 1. row statistics

template <int DT, bool VEC>
__global__ __launch_bounds__(kThreads) void k_rowstats(Params P) {
  using U = Unit<DT, VEC>;
  constexpr int W = U::W;
  __shared__ float shf[kWaves];
  __shared__ double shd[kWaves];
  __shared__ int32_t shi[kWaves];

  const int64_t wg = blockIdx.x;
  const int32_t split = (int32_t)(wg % P.nsplit);
  const int64_t slot = wg / P.nsplit;
  const int32_t b = (int32_t)(slot / P.spr);
  const int32_t k = (int32_t)(slot % P.spr);
  int64_t dbase;
  int32_t gb;
  float T;
  request(P, b, dbase, gb, T);
  const bool sampling = T > 0.f;

  const void *base;
  int64_t row;
  if (k <= P.gamma) {
    if (k > gb) return;
    base = P.target;
    row = dbase + b + k;
  } else {
    const int32_t i = k - P.gamma - 1;
    if (i >= gb || !sampling) return;
    base = P.draft;
    row = dbase + i;
  }
  const void *rp = row_ptr<DT>(base, row, P.V);
  const int64_t lo = (int64_t)split * P.split_len;
  const int64_t hi = lo + P.split_len < P.V ? lo + P.split_len : P.V;
  const int64_t u0 = lo / W, u1 = hi > lo ? hi / W : u0;  // lo, hi are multiples of W
  Partial *out = P.parts + slot * P.nsplit + split;
  const int tid = threadIdx.x;

  if (sampling) {
    const TempConst tc = temp_const(T);
    float m = -INFINITY;
    double s = 0.0;
    for (int64_t ub = u0; ub < u1; ub += (int64_t)kThreads * kUnroll) {
      if (ub + tid >= u1) break;
      float x[kUnroll][W];
      bool ok[kUnroll];
#pragma unroll
      for (int j = 0; j < kUnroll; ++j) {
        const int64_t u = ub + (int64_t)j * kThreads + tid;
        ok[j] = u < u1;
        if (ok[j]) {
          U::load(rp, u, x[j]);
        } else {
#pragma unroll
          for (int e = 0; e < W; ++e) x[j][e] = -INFINITY;
        }
      }
      float cm = m;
#pragma unroll
      for (int j = 0; j < kUnroll; ++j)
#pragma unroll
        for (int e = 0; e < W; ++e) cm = fmaxf(cm, x[j][e]);
      if (cm > m) {
        s *= exp2(((double)m - (double)cm) * tc.c);
        m = cm;
      }
#pragma unroll
      for (int j = 0; j < kUnroll; ++j) {
#pragma unroll
        for (int e = 0; e < W; ++e) {
          const float t = exp_term(x[j][e], m, tc.c_hi, tc.c_lo);
          s += ok[j] ? (double)t : 0.0;
        }
      }
    }
    const float M = block_max(m, shf);
    const double scaled = (m == -INFINITY) ? 0.0 : s * exp2(((double)m - (double)M) * tc.c);
    const double S = block_sum(scaled, shd);
    if (tid == 0) {
      out->m = M;
      out->idx = 0;
      out->s = S;
    }
  } else {
    float bv = -INFINITY;
    int32_t bi = INT32_MAX;
    for (int64_t ub = u0; ub < u1; ub += (int64_t)kThreads * kUnroll) {
      if (ub + tid >= u1) break;
#pragma unroll
      for (int j = 0; j < kUnroll; ++j) {
        const int64_t u = ub + (int64_t)j * kThreads + tid;
        if (u < u1) {
          float x[W];
          U::load(rp, u, x);
#pragma unroll
          for (int e = 0; e < W; ++e) {
            if (x[e] > bv) {
              bv = x[e];
              bi = (int32_t)(u * W + e);
            }
          }
        }
      }
    }
    block_argmax(bv, bi, shf, shi);
    if (tid == 0) {
      out->m = bv;
      out->idx = bi;
      out->s = 0.0;
    }
  }
}

// ------------------------------------------------------------------ 2. decide

__device__ void merge_stats(const Params &P, int64_t slot, double c, double &m, double &s) {
  const Partial *pp = P.parts + slot * P.nsplit;
  float mx = -INFINITY;
  for (int i = 0; i < P.nsplit; ++i) mx = fmaxf(mx, pp[i].m);
  double acc = 0.0;
  for (int i = 0; i < P.nsplit; ++i) {
    const Partial q = pp[i];
    if (q.m != -INFINITY) acc += q.s * exp2(((double)q.m - (double)mx) * c);
  }
  m = mx;
  s = acc;
}

__device__ void merge_argmax(const Params &P, int64_t slot, float &bv, int32_t &bi) {
  const Partial *pp = P.parts + slot * P.nsplit;
  bv = -INFINITY;
  bi = INT32_MAX;
  for (int i = 0; i < P.nsplit; ++i) argmax_merge(bv, bi, pp[i].m, pp[i].idx);
}

template <int DT>
__global__ __launch_bounds__(kThreads) void k_decide(Params P) {
  const int lane = threadIdx.x & 63;
  const int32_t b = (int32_t)(blockIdx.x * kWaves + (threadIdx.x >> 6));
  if (b >= P.B) return;
  int64_t dbase;
  int32_t gb;
  float T;
  request(P, b, dbase, gb, T);
  const int64_t tbase = dbase + b;
  const bool sampling = T > 0.f;
  const int64_t slot0 = (int64_t)b * P.spr;
  const int64_t dslot0 = slot0 + P.gamma + 1;
  const TempConst tc = temp_const(sampling ? T : 1.f);

  bool accept = false;
  if (lane < gb) {
    const int32_t x = P.tokens[dbase + lane];
    if (!sampling) {
      float bv;
      int32_t bi;
      merge_argmax(P, slot0 + lane, bv, bi);
      accept = x == bi;
    } else {
      double mt, st, md, sd;
      merge_stats(P, slot0 + lane, tc.c, mt, st);
      merge_stats(P, dslot0 + lane, tc.c, md, sd);
      double p = 0.0, q = 0.0;
      if (x >= 0 && x < P.V) {
        const double zt = logit_at<DT>(P.target, (tbase + lane) * P.V + x);
        const double zd = logit_at<DT>(P.draft, (dbase + lane) * P.V + x);
        p = exp2((zt - mt) * tc.c) / st;
        q = exp2((zd - md) * tc.c) / sd;
      }
      const double u = (double)P.uniforms[2 * (tbase + lane)];
      accept = u * q < p;
      if (P.p_x) P.p_x[dbase + lane] = p;
      if (P.q_x) P.q_x[dbase + lane] = q;
    }
  }
  const uint64_t acc_mask = __ballot(accept);
  const uint64_t valid = gb >= 64 ? ~0ull : ((1ull << gb) - 1ull);
  const uint64_t rej = ~acc_mask & valid;
  const int32_t j = rej ? (int32_t)(__ffsll((long long)rej) - 1) : gb;

  for (int32_t i = lane; i <= gb; i += 64) {
    if (i != j) P.out_tokens[tbase + i] = i < j ? P.tokens[dbase + i] : -1;
  }
  if (lane == 0) {
    P.out_n[b] = j;
    Stop st = {};
    st.j = j;
    if (!sampling) {
      float bv;
      int32_t bi;
      merge_argmax(P, slot0 + j, bv, bi);
      P.out_tokens[tbase + j] = bi;
      st.mode = kModeNone;
    } else {
      double mt, s_t;
      merge_stats(P, slot0 + j, tc.c, mt, s_t);
      st.mt = (float)mt;
      st.st = s_t;
      st.c = tc.c;
      st.c_hi = tc.c_hi;
      st.c_lo = tc.c_lo;
      if (j < gb) {
        double md, s_d;
        merge_stats(P, dslot0 + j, tc.c, md, s_d);
        st.md = (float)md;
        st.sd = s_d;
        st.k = (mt - md) * tc.c + log2(s_t / s_d);
        st.mode = kModeResidual;
      } else {
        st.mode = kModeBonus;
      }
    }
    P.stop[b] = st;
  }

  // Diagnostics.
  if (P.row_max_t || P.row_sum_t) {
    for (int32_t i = lane; i <= gb; i += 64) {
      if (sampling) {
        double m, s;
        merge_stats(P, slot0 + i, tc.c, m, s);
        if (P.row_max_t) P.row_max_t[tbase + i] = (float)m;
        if (P.row_sum_t) P.row_sum_t[tbase + i] = s;
      } else if (P.row_max_t) {
        float bv;
        int32_t bi;
        merge_argmax(P, slot0 + i, bv, bi);
        P.row_max_t[tbase + i] = bv;
      }
    }
  }
  if (sampling && (P.row_max_d || P.row_sum_d)) {
    for (int32_t i = lane; i < gb; i += 64) {
      double m, s;
      merge_stats(P, dslot0 + i, tc.c, m, s);
      if (P.row_max_d) P.row_max_d[dbase + i] = (float)m;
      if (P.row_sum_d) P.row_sum_d[dbase + i] = s;
    }
  }
}

// ------------------------------------------------------------------ 3. residual mass

// Unnormalised weight of token k at the stop row: S_t * max(p_k - q_k, 0), or S_t * p_k.
template <int MODE>
__device__ __forceinline__ float resid_weight(float zt, float zd, const Stop &st) {
  const float et = exp_term(zt, st.mt, st.c_hi, st.c_lo);
  if constexpr (MODE == kModeBonus) {
    return et;
  } else {
    const double delta = ((double)zd - (double)zt) * st.c + st.k;  // log2(q_k / p_k)
    if (!(delta < 0.0)) return 0.f;
    return et * -expm1f((float)(delta * kLn2));
  }
}

template <int DT, bool VEC, int MODE>
__device__ double resid_range_sum(const void *tr, const void *dr, int64_t u0, int64_t u1,
                                  const Stop &st) {
  using U = Unit<DT, VEC>;
  constexpr int W = U::W;
  double acc = 0.0;
  for (int64_t u = u0 + threadIdx.x; u < u1; u += kThreads) {
    float zt[W], zd[W];
    U::load(tr, u, zt);
    if constexpr (MODE == kModeResidual) U::load(dr, u, zd);
#pragma unroll
    for (int e = 0; e < W; ++e)
      acc += (double)resid_weight<MODE>(zt[e], MODE == kModeResidual ? zd[e] : 0.f, st);
  }
  return acc;
}

template <int DT, bool VEC>
__global__ __launch_bounds__(kThreads) void k_resid(Params P) {
  constexpr int W = Unit<DT, VEC>::W;
  __shared__ double shd[kWaves];
  const int64_t wg = blockIdx.x;
  const int32_t b = (int32_t)(wg / P.nsplit_r);
  const int32_t split = (int32_t)(wg % P.nsplit_r);
  const Stop st = P.stop[b];
  if (st.mode == kModeNone) return;
  int64_t dbase;
  int32_t gb;
  float T;
  request(P, b, dbase, gb, T);
  const void *tr = row_ptr<DT>(P.target, dbase + b + st.j, P.V);
  const void *dr = row_ptr<DT>(P.draft, dbase + st.j, P.V);
  const int64_t lo = (int64_t)split * P.split_len_r;
  const int64_t hi = lo + P.split_len_r < P.V ? lo + P.split_len_r : P.V;
  const int64_t u0 = lo / W, u1 = hi > lo ? hi / W : u0;
  double acc = st.mode == kModeResidual
                   ? resid_range_sum<DT, VEC, kModeResidual>(tr, dr, u0, u1, st)
                   : resid_range_sum<DT, VEC, kModeBonus>(tr, dr, u0, u1, st);
  acc = block_sum(acc, shd);
  if (threadIdx.x == 0) P.rsum[(int64_t)b * P.nsplit_r + split] = acc;
}

// ------------------------------------------------------------------ 4. draw

// Inverse CDF inside units [u0, u1) of the stop row: each thread owns a contiguous run of
// units; a block scan of the run totals picks the thread, which then walks its run.
// If `frac` is set, the target is u * (total of the range); otherwise it is `target`.
template <int DT, bool VEC, int MODE>
__device__ int32_t draw_in_range(const void *tr, const void *dr, int64_t u0, int64_t u1,
                                 const Stop &st, double target, bool frac, double u,
                                 double &range_total) {
  using U = Unit<DT, VEC>;
  constexpr int W = U::W;
  __shared__ double shs[kWaves];
  __shared__ int32_t sh_first[kWaves], sh_last[kWaves];
  const int tid = threadIdx.x;
  const int64_t n = u1 - u0;
  const int64_t per = (n + kThreads - 1) / kThreads;
  const int64_t a = u0 + tid * per;
  const int64_t e_ = a + per < u1 ? a + per : u1;

  double mine = 0.0;
  for (int64_t uu = a; uu < e_; ++uu) {
    float zt[W], zd[W];
    U::load(tr, uu, zt);
    if constexpr (MODE == kModeResidual) U::load(dr, uu, zd);
#pragma unroll
    for (int e = 0; e < W; ++e)
      mine += (double)resid_weight<MODE>(zt[e], MODE == kModeResidual ? zd[e] : 0.f, st);
  }
  double total;
  const double before = block_exclusive_scan(mine, shs, total);
  range_total = total;
  if (frac) target = u * total;

  // first thread whose run crosses the target; last thread with positive mass
  const bool crosses = mine > 0.0 && before + mine > target;
  const uint64_t cm = __ballot(crosses), pm = __ballot(mine > 0.0);
  const int w = tid >> 6;
  if ((tid & 63) == 0) {
    sh_first[w] = cm ? w * 64 + __ffsll((long long)cm) - 1 : INT32_MAX;
    sh_last[w] = pm ? w * 64 + 63 - __clzll((long long)pm) : -1;
  }
  __syncthreads();
  int32_t first = INT32_MAX, last = -1;
  for (int i = 0; i < kWaves; ++i) {
    first = sh_first[i] < first ? sh_first[i] : first;
    last = sh_last[i] > last ? sh_last[i] : last;
  }
  __syncthreads();
  const int32_t pick = first != INT32_MAX ? first : last;
  const bool exact = first != INT32_MAX;
  int32_t result = -1;
  if (pick >= 0 && tid == pick) {
    double run = before;
    int32_t last_pos = -1;
    for (int64_t uu = a; uu < e_ && result < 0; ++uu) {
      float zt[W], zd[W];
      U::load(tr, uu, zt);
      if constexpr (MODE == kModeResidual) U::load(dr, uu, zd);
#pragma unroll
      for (int e = 0; e < W; ++e) {
        const float r = resid_weight<MODE>(zt[e], MODE == kModeResidual ? zd[e] : 0.f, st);
        run += (double)r;
        if (r > 0.f) {
          last_pos = (int32_t)(uu * W + e);
          if (exact && result < 0 && run > target) result = last_pos;
        }
      }
    }
    if (result < 0) result = last_pos;
  }
  return result;  // valid in thread `pick` only; -1 elsewhere
}

template <int DT, bool VEC>
__global__ __launch_bounds__(kThreads) void k_sample(Params P) {
  constexpr int W = Unit<DT, VEC>::W;
  __shared__ double sh_target, sh_R;
  __shared__ int32_t sh_split, sh_token;
  const int32_t b = blockIdx.x;
  const Stop st = P.stop[b];
  if (st.mode == kModeNone) return;
  int64_t dbase;
  int32_t gb;
  float T;
  request(P, b, dbase, gb, T);
  const int64_t tbase = dbase + b;
  const void *tr = row_ptr<DT>(P.target, tbase + st.j, P.V);
  const void *dr = row_ptr<DT>(P.draft, dbase + st.j, P.V);
  const double u = (double)P.uniforms[2 * (tbase + st.j) + 1];
  const double *rs = P.rsum + (int64_t)b * P.nsplit_r;

  if (threadIdx.x == 0) {
    double R = 0.0;
    for (int s = 0; s < P.nsplit_r; ++s) R += rs[s];
    const double target = u * R;
    double C = 0.0;
    int32_t pick = -1, last = -1;
    double local = 0.0;
    for (int s = 0; s < P.nsplit_r; ++s) {
      const double r = rs[s];
      if (r > 0.0) {
        last = s;
        if (C + r > target) {
          pick = s;
          local = target - C;
          break;
        }
      }
      C += r;
    }
    if (pick < 0 && last >= 0) {  // u >= 1 or rounding at the very end: last positive slice
      pick = last;
      local = INFINITY;
    }
    sh_split = pick;
    sh_target = local;
    sh_R = R;
    sh_token = -1;
  }
  __syncthreads();
  const int32_t split = sh_split;
  double range_total = 0.0;
  int32_t tok;
  double mass;
  if (split >= 0) {
    const int64_t lo = (int64_t)split * P.split_len_r;
    const int64_t hi = lo + P.split_len_r < P.V ? lo + P.split_len_r : P.V;
    tok = st.mode == kModeResidual
              ? draw_in_range<DT, VEC, kModeResidual>(tr, dr, lo / W, hi / W, st, sh_target,
                                                      false, u, range_total)
              : draw_in_range<DT, VEC, kModeBonus>(tr, dr, lo / W, hi / W, st, sh_target,
                                                   false, u, range_total);
    mass = sh_R / st.st;
  } else {
    // Empty residual (p <= q everywhere after rounding): draw from p_j over the whole row.
    tok = draw_in_range<DT, VEC, kModeBonus>(tr, dr, 0, P.V / W, st, 0.0, true, u,
                                             range_total);
    mass = range_total / st.st;
  }
  if (tok >= 0) sh_token = tok;
  __syncthreads();
  if (threadIdx.x == 0) {
    P.out_tokens[tbase + st.j] = sh_token;
    if (P.resid_mass) P.resid_mass[b] = mass;
  }
}

// ------------------------------------------------------------------ host side

struct Plan {
  int32_t spr, nsplit, nsplit_r;
  int64_t split_len, split_len_r;
  size_t off_parts, off_stop, off_rsum, total;
};

size_t align_up(size_t x) { return (x + kAlign - 1) / kAlign * kAlign; }

// Slices per row: at least one full pass of the block's loads per slice where V allows,
// more slices when there are too few rows to give every CU work.
void choose_splits(int64_t rows, int64_t V, int W, int32_t &nsplit, int64_t &split_len) {
  const int64_t units = (V + W - 1) / W;
  int64_t ns = (units + (int64_t)kThreads * kUnroll - 1) / ((int64_t)kThreads * kUnroll);
  if (rows * ns < kTargetWorkgroups) ns = (kTargetWorkgroups + rows - 1) / rows;
  const int64_t cap = units / kMinUnitsPerSplit > 1 ? units / kMinUnitsPerSplit : 1;
  if (ns > cap) ns = cap;
  if (ns > kMaxSplits) ns = kMaxSplits;
  if (ns < 1) ns = 1;
  const int64_t per = (units + ns - 1) / ns;
  ns = (units + per - 1) / per;  // no empty slice
  nsplit = (int32_t)ns;
  split_len = per * W;
}

bool make_plan(int32_t B, int32_t gamma, int64_t V, int dtype, bool greedy, Plan &pl) {
  if (B < 0 || gamma < 0 || gamma > SPEC_MAX_GAMMA || V < 1 || V > INT32_MAX) return false;
  if (dtype != SPEC_F32 && dtype != SPEC_BF16) return false;
  const int W = dtype == SPEC_F32 ? 4 : 8;
  pl.spr = greedy ? gamma + 1 : 2 * gamma + 1;
  const int64_t bb = B > 0 ? B : 1;
  choose_splits(bb * pl.spr, V, W, pl.nsplit, pl.split_len);
  choose_splits(bb * 2, V, W, pl.nsplit_r, pl.split_len_r);
  pl.off_parts = 0;
  pl.off_stop = align_up((size_t)bb * pl.spr * pl.nsplit * sizeof(Partial));
  pl.off_rsum = pl.off_stop + align_up((size_t)bb * sizeof(Stop));
  pl.total = pl.off_rsum + align_up((size_t)bb * pl.nsplit_r * sizeof(double));
  return true;
}

int record(const spec_probe *probe, int k, hipStream_t s) {
  if (!probe || !probe->events[k]) return SPEC_OK;
  return hipEventRecord((hipEvent_t)probe->events[k], s) == hipSuccess ? SPEC_OK
                                                                       : SPEC_ERR_HIP;
}

#define SPEC_TRY(expr)            \
  do {                            \
    const int rc_ = (expr);       \
    if (rc_ != SPEC_OK) return rc_; \
  } while (0)

int launched() { return hipGetLastError() == hipSuccess ? SPEC_OK : SPEC_ERR_HIP; }

template <int DT, bool VEC>
int run_sample(const Params &P, const Plan &pl, const spec_probe *probe, hipStream_t s) {
  const int64_t g1 = (int64_t)P.B * pl.spr * pl.nsplit;
  const int64_t g3 = (int64_t)P.B * pl.nsplit_r;
  SPEC_TRY(record(probe, 0, s));
  k_rowstats<DT, VEC><<<dim3((uint32_t)g1), dim3(kThreads), 0, s>>>(P);
  SPEC_TRY(launched());
  SPEC_TRY(record(probe, 1, s));
  SPEC_TRY(record(probe, 2, s));
  k_decide<DT><<<dim3((uint32_t)((P.B + kWaves - 1) / kWaves)), dim3(kThreads), 0, s>>>(P);
  SPEC_TRY(launched());
  SPEC_TRY(record(probe, 3, s));
  SPEC_TRY(record(probe, 4, s));
  k_resid<DT, VEC><<<dim3((uint32_t)g3), dim3(kThreads), 0, s>>>(P);
  SPEC_TRY(launched());
  SPEC_TRY(record(probe, 5, s));
  SPEC_TRY(record(probe, 6, s));
  k_sample<DT, VEC><<<dim3((uint32_t)P.B), dim3(kThreads), 0, s>>>(P);
  SPEC_TRY(launched());
  SPEC_TRY(record(probe, 7, s));
  return SPEC_OK;
}

template <int DT, bool VEC>
int run_greedy(const Params &P, const Plan &pl, const spec_probe *probe, hipStream_t s) {
  const int64_t g1 = (int64_t)P.B * pl.spr * pl.nsplit;
  SPEC_TRY(record(probe, 0, s));
  k_rowstats<DT, VEC><<<dim3((uint32_t)g1), dim3(kThreads), 0, s>>>(P);
  SPEC_TRY(launched());
  SPEC_TRY(record(probe, 1, s));
  SPEC_TRY(record(probe, 2, s));
  k_decide<DT><<<dim3((uint32_t)((P.B + kWaves - 1) / kWaves)), dim3(kThreads), 0, s>>>(P);
  SPEC_TRY(launched());
  SPEC_TRY(record(probe, 3, s));
  return SPEC_OK;
}

bool aligned16(const void *p) { return ((uintptr_t)p & 15u) == 0; }

int common_checks(int32_t B, int32_t gamma, int64_t V, int dtype, void *workspace,
                  size_t workspace_bytes, const Plan &pl, int64_t grid1) {
  (void)B; (void)gamma; (void)V; (void)dtype;
  if (!workspace) return SPEC_ERR_NULL;
  if (((uintptr_t)workspace & (kAlign - 1)) != 0 || workspace_bytes < pl.total)
    return SPEC_ERR_WORKSPACE;
  if (grid1 > (int64_t)UINT32_MAX) return SPEC_ERR_SHAPE;
  return SPEC_OK;
}

void fill_workspace(Params &P, const Plan &pl, void *workspace) {
  char *ws = static_cast<char *>(workspace);
  P.parts = reinterpret_cast<Partial *>(ws + pl.off_parts);
  P.stop = reinterpret_cast<Stop *>(ws + pl.off_stop);
  P.rsum = reinterpret_cast<double *>(ws + pl.off_rsum);
  P.spr = pl.spr;
  P.nsplit = pl.nsplit;
  P.split_len = pl.split_len;
  P.nsplit_r = pl.nsplit_r;
  P.split_len_r = pl.split_len_r;
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
    case SPEC_ERR_SHAPE: return "invalid sizes (B < 0, gamma outside [0, 64], V outside [1, 2^31-1], or grid too large)";
    case SPEC_ERR_DTYPE: return "dtype is neither SPEC_F32 nor SPEC_BF16";
    case SPEC_ERR_WORKSPACE: return "workspace too small or not 256-byte aligned";
    case SPEC_ERR_HIP: return "HIP kernel launch or event record failed";
    default: return "unknown spec_verify error code";
  }
}

int spec_verify_sample(const void *target_logits, const void *draft_logits, int dtype,
                       const int32_t *draft_tokens, const float *uniforms,
                       const float *temperatures, int32_t B, int32_t gamma,
                       const int32_t *cu_draft, int64_t V, int32_t *out_tokens,
                       int32_t *out_num_accepted, void *workspace, size_t workspace_bytes,
                       const spec_probe *probe, void *stream) {
  if (dtype != SPEC_F32 && dtype != SPEC_BF16) return SPEC_ERR_DTYPE;
  if (B < 0 || gamma < 0 || gamma > SPEC_MAX_GAMMA || V < 1 || V > INT32_MAX)
    return SPEC_ERR_SHAPE;
  if (B == 0) return SPEC_OK;
  if (!target_logits || !draft_logits || !draft_tokens || !uniforms || !temperatures ||
      !out_tokens || !out_num_accepted)
    return SPEC_ERR_NULL;
  Plan pl;
  if (!make_plan(B, gamma, V, dtype, false, pl)) return SPEC_ERR_SHAPE;
  const int64_t grid1 = (int64_t)B * pl.spr * pl.nsplit;
  SPEC_TRY(common_checks(B, gamma, V, dtype, workspace, workspace_bytes, pl, grid1));
  if ((int64_t)B * pl.nsplit_r > (int64_t)UINT32_MAX) return SPEC_ERR_SHAPE;

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
  fill_workspace(P, pl, workspace);
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
  if (dtype == SPEC_F32)
    return vec ? run_sample<SPEC_F32, true>(P, pl, probe, s)
               : run_sample<SPEC_F32, false>(P, pl, probe, s);
  return vec ? run_sample<SPEC_BF16, true>(P, pl, probe, s)
             : run_sample<SPEC_BF16, false>(P, pl, probe, s);
}

int spec_verify_greedy(const void *target_logits, int dtype, const int32_t *draft_tokens,
                       int32_t B, int32_t gamma, const int32_t *cu_draft, int64_t V,
                       int32_t *out_tokens, int32_t *out_num_accepted, void *workspace,
                       size_t workspace_bytes, const spec_probe *probe, void *stream) {
  if (dtype != SPEC_F32 && dtype != SPEC_BF16) return SPEC_ERR_DTYPE;
  if (B < 0 || gamma < 0 || gamma > SPEC_MAX_GAMMA || V < 1 || V > INT32_MAX)
    return SPEC_ERR_SHAPE;
  if (B == 0) return SPEC_OK;
  if (!target_logits || !draft_tokens || !out_tokens || !out_num_accepted)
    return SPEC_ERR_NULL;
  Plan pl;
  if (!make_plan(B, gamma, V, dtype, true, pl)) return SPEC_ERR_SHAPE;
  const int64_t grid1 = (int64_t)B * pl.spr * pl.nsplit;
  SPEC_TRY(common_checks(B, gamma, V, dtype, workspace, workspace_bytes, pl, grid1));

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
  fill_workspace(P, pl, workspace);
  if (probe) P.row_max_t = probe->row_max_t;
  const int es = dtype == SPEC_F32 ? 4 : 2;
  const bool vec = aligned16(target_logits) && (V * es) % 16 == 0;
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (dtype == SPEC_F32)
    return vec ? run_greedy<SPEC_F32, true>(P, pl, probe, s)
               : run_greedy<SPEC_F32, false>(P, pl, probe, s);
  return vec ? run_greedy<SPEC_BF16, true>(P, pl, probe, s)
             : run_greedy<SPEC_BF16, false>(P, pl, probe, s);
}

}  // extern "C"
