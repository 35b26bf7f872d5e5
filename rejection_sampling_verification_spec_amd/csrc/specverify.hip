// specverify.hip -- the verify step of speculative sampling (modified rejection
// sampling) as hand-written HIP kernels for CDNA4 (gfx950, wave64), behind the
// C ABI declared in include/specverify.h.
//
// The method (reference pages):
//   [P1] "Speculative Decoding（投機的デコーディング）— 小さなモデルでLLM推論を高速化する"
//        sections ステップ3: 受理・棄却判定, 修正分布の定義, Pythonによるシミュレーション実装
//   [P2] "論文解説: Fast Inference from Transformers via Speculative Decoding"
//        sections 投機的サンプリングアルゴリズム (accept and modified-distribution
//        equations), 実装のポイント (greedy)
//   [P3] "投機的デコーディングとは：同時リクエストが多いと遅くなる理由"
//        section 先読みは、一回の順伝播で進むトークンを増やす (greedy worked example)
//   [P4] "LLM推測デコーディング最適化実踐", section 検証アルゴリズムの実装
//        (gamma+1 target rows, bonus draw from the last one)
//
// Three launches on the caller's stream, no host synchronisation:
//
//   K1 row_stats   one workgroup per (request, logit row, vocabulary tile).
//                  Streams the tile once with 16-byte loads and produces, for a
//                  stochastic row, (M, s) with M an integer upper bound of
//                  max(z)*log2(e)/T and s = sum 2^(z*c - M); for a greedy row,
//                  the maximum and its lowest index.  The integer M makes every
//                  rescale between partial sums an exact power of two (ldexp).
//   K2 decide      one workgroup per request.  Merges the tile partials of each
//                  row in a fixed order, evaluates a_i = min(1, p_i(x_i)/q_i(x_i))
//                  in fp64 from the two gathered logits, finds the first
//                  rejection with a wave ballot, writes accepted_count and the
//                  accepted prefix, and prepares the one row pair to sample.
//   K3 sample      B x NW workgroups.  Re-reads the selected target row (and
//                  draft row after a rejection), forms w = max(0, p - q) (or p
//                  for the bonus), writes one fp64 mass per 512-token sub-chunk,
//                  and the last workgroup of each request to finish finds u*Z by
//                  a scan over the sub-chunk masses and then inside the one
//                  sub-chunk that holds it.
//
// Numerics: bf16 -> fp32 widening is exact; exponentials are v_exp_f32 of
// fma(z, c, -M); per-thread partial sums are fp32 over at most 64 terms and
// everything above a thread (wave, workgroup, tile, CDF prefix) is fp64.
#include <hip/hip_runtime.h>

#include <math.h>
#include <stdint.h>
#include <string.h>

#include "specverify.h"

namespace {

constexpr int kBlock = 256;          // threads per workgroup (4 waves of 64)
constexpr int kWave = 64;
constexpr int kWaves = kBlock / kWave;
constexpr int kSub = 512;            // tokens per K3 sub-chunk (64 lanes x 8)
constexpr int kEmptyM = -(1 << 28);  // exponent of an empty partial
constexpr double kLog2e = 1.4426950408889634073599246810019;
constexpr size_t kAlign = 256;

// ------------------------------------------------------------------ elements
template <int DT> struct Elem;
template <> struct Elem<SV_F32> {
  static constexpr int kVec = 4;    // elements per 16-byte vector
  static constexpr int kBytes = 4;
};
template <> struct Elem<SV_BF16> {
  static constexpr int kVec = 8;
  static constexpr int kBytes = 2;
};

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

template <int DT>
__device__ __forceinline__ float load_one(const void *row, long e) {
  if constexpr (DT == SV_F32) {
    return static_cast<const float *>(row)[e];
  } else {
    return __uint_as_float(static_cast<uint32_t>(static_cast<const uint16_t *>(row)[e]) << 16);
  }
}

// One aligned 16-byte vector starting at element e0.
template <int DT>
__device__ __forceinline__ void load_vec(const void *row, long e0, float *x) {
  const uint4 v = *reinterpret_cast<const uint4 *>(static_cast<const char *>(row) +
                                                   e0 * Elem<DT>::kBytes);
  if constexpr (DT == SV_F32) {
    x[0] = __uint_as_float(v.x);
    x[1] = __uint_as_float(v.y);
    x[2] = __uint_as_float(v.z);
    x[3] = __uint_as_float(v.w);
  } else {
    x[0] = bf16_lo(v.x);
    x[1] = bf16_hi(v.x);
    x[2] = bf16_lo(v.y);
    x[3] = bf16_hi(v.y);
    x[4] = bf16_lo(v.z);
    x[5] = bf16_hi(v.z);
    x[6] = bf16_lo(v.w);
    x[7] = bf16_hi(v.w);
  }
}

// kVec elements starting at e0; elements at or beyond `end` read as -inf.
template <int DT>
__device__ __forceinline__ void load_vec_guarded(const void *row, bool aligned, long e0, long end,
                                                 float *x) {
  constexpr int kV = Elem<DT>::kVec;
  if (aligned && e0 + kV <= end) {
    load_vec<DT>(row, e0, x);
  } else {
#pragma unroll
    for (int e = 0; e < kV; ++e) x[e] = (e0 + e < end) ? load_one<DT>(row, e0 + e) : -INFINITY;
  }
}

// ------------------------------------------------------------------ temperature
// c = log2(e) / T rounded once to fp32; every kernel derives it the same way.
__device__ __forceinline__ float temp_scale(float T) {
  return static_cast<float>(kLog2e / static_cast<double>(T));
}

__device__ __forceinline__ float request_T(const float *temps, float scalar_T, int b) {
  return temps ? temps[b] : scalar_T;
}

// Draft length of request b, clamped to [0, gamma] so that no row outside the
// padded layout is ever addressed.
__device__ __forceinline__ int request_len(const int32_t *lens, int gamma, int b) {
  if (!lens) return gamma;
  const int g = lens[b];
  return g < 0 ? 0 : (g > gamma ? gamma : g);
}

// ------------------------------------------------------------------ partials
// One 16-byte record per (request, row, tile).  Stochastic rows: s and M (and
// the tile max for diagnostics).  Greedy rows: the max and its index.
struct alignas(16) Partial {
  double s;
  float mx;
  int mi;  // M (stochastic) or arg-max index (greedy)
};

__device__ __forceinline__ void merge_sm(int &M, double &s, float &mx, int Mo, double so, float mo) {
  const int Mn = M > Mo ? M : Mo;
  s = ldexp(s, M - Mn) + ldexp(so, Mo - Mn);  // exact rescale by powers of two
  M = Mn;
  mx = fmaxf(mx, mo);
}

__device__ __forceinline__ void merge_arg(float &v, int &i, float vo, int io) {
  if (vo > v || (vo == v && io < i)) {
    v = vo;
    i = io;
  }
}

// Per-request parameters of the sampling step (written by K2, read by K3).
struct alignas(16) SelParams {
  int mode;      // 0: nothing to sample (greedy), 1: residual at k, 2: bonus at k
  int k;         // position sampled
  float c;       // log2(e)/T
  float negMp;   // -M of target row k
  float negMq;   // -M of draft row k
  float r;       // s'_p / s'_q: residual in units of the target row's scale
  double ip;     // 1 / s'_p (only for the diagnostic residual mass)
};

struct alignas(16) SubSums {
  double w;  // sum of w over the sub-chunk (target-row units)
  double p;  // sum of 2^(z_p c - M_p) over the sub-chunk (zero-mass fallback)
};

// ================================================================== K1
// Rows of request b: r in [0, gamma] are target rows, r in [gamma+1, 2 gamma]
// are draft rows r - gamma - 1.  A row is needed if it is a target row i <= g_b,
// or a draft row i < g_b of a stochastic request (greedy requests never read
// draft logits).
template <int DT, int U>
__global__ __launch_bounds__(kBlock) void k1_row_stats(
    const void *__restrict__ target, const void *__restrict__ draft,
    const float *__restrict__ temps, float scalar_T, const int32_t *__restrict__ lens, int gamma,
    int V, int NS, Partial *__restrict__ part) {
  constexpr int kV = Elem<DT>::kVec;
  constexpr long kTile = static_cast<long>(kBlock) * U * kV;
  const int rows = 2 * gamma + 1;
  const long tile = blockIdx.x;
  const int j = static_cast<int>(tile % NS);
  const long slot = tile / NS;
  const int r = static_cast<int>(slot % rows);
  const int b = static_cast<int>(slot / rows);
  const int g = request_len(lens, gamma, b);
  const float T = request_T(temps, scalar_T, b);
  const bool is_target = r <= gamma;
  const int i = is_target ? r : r - gamma - 1;
  const bool greedy = !(T > 0.0f);
  if (is_target ? (i > g) : (greedy || i >= g)) return;

  const void *row =
      is_target
          ? static_cast<const void *>(static_cast<const char *>(target) +
                                      (static_cast<long>(b) * (gamma + 1) + i) * V * Elem<DT>::kBytes)
          : static_cast<const void *>(static_cast<const char *>(draft) +
                                      (static_cast<long>(b) * gamma + i) * V * Elem<DT>::kBytes);
  const bool aligned = (reinterpret_cast<uintptr_t>(row) & 15u) == 0;
  const long t0 = j * kTile;
  const long t1 = (t0 + kTile < V) ? t0 + kTile : V;
  const int tid = threadIdx.x;

  float x[U][kV];
  if (aligned && t1 - t0 == kTile) {
#pragma unroll
    for (int u = 0; u < U; ++u) load_vec<DT>(row, t0 + static_cast<long>(tid + u * kBlock) * kV, x[u]);
  } else {
#pragma unroll
    for (int u = 0; u < U; ++u)
      load_vec_guarded<DT>(row, aligned, t0 + static_cast<long>(tid + u * kBlock) * kV, t1, x[u]);
  }

  __shared__ double sh_s[kWaves];
  __shared__ float sh_mx[kWaves];
  __shared__ int sh_mi[kWaves];
  const int lane = tid & (kWave - 1);
  const int wave = tid / kWave;

  if (!greedy) {
    const float c = temp_scale(T);
    float mx = -INFINITY;
#pragma unroll
    for (int u = 0; u < U; ++u)
#pragma unroll
      for (int e = 0; e < kV; ++e) mx = fmaxf(mx, x[u][e]);
    int M = kEmptyM;
    double s = 0.0;
    if (mx > -INFINITY) {
      const float Mf = ceilf(mx * c);
      M = static_cast<int>(Mf);
      const float nM = -Mf;
      float acc[kV];
#pragma unroll
      for (int e = 0; e < kV; ++e) acc[e] = 0.0f;
#pragma unroll
      for (int u = 0; u < U; ++u)
#pragma unroll
        for (int e = 0; e < kV; ++e) acc[e] += __builtin_amdgcn_exp2f(fmaf(x[u][e], c, nM));
#pragma unroll
      for (int w = kV / 2; w >= 1; w /= 2)
#pragma unroll
        for (int e = 0; e < w; ++e) acc[e] += acc[e + w];
      s = static_cast<double>(acc[0]);
    }
#pragma unroll
    for (int off = kWave / 2; off >= 1; off /= 2) {
      const int Mo = __shfl_xor(M, off);
      const double so = __shfl_xor(s, off);
      const float mo = __shfl_xor(mx, off);
      merge_sm(M, s, mx, Mo, so, mo);
    }
    if (lane == 0) {
      sh_s[wave] = s;
      sh_mx[wave] = mx;
      sh_mi[wave] = M;
    }
    __syncthreads();
    if (tid == 0) {
      int Mt = sh_mi[0];
      double st = sh_s[0];
      float mt = sh_mx[0];
      for (int w = 1; w < kWaves; ++w) merge_sm(Mt, st, mt, sh_mi[w], sh_s[w], sh_mx[w]);
      Partial pr;
      pr.s = st;
      pr.mx = mt;
      pr.mi = Mt;
      part[tile] = pr;
    }
  } else {
    // lowest index of the maximum (fp32 compare; bf16 widening is exact)
    float bv = -INFINITY;
    int bi = 0x7fffffff;
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const long e0 = t0 + static_cast<long>(tid + u * kBlock) * kV;
#pragma unroll
      for (int e = 0; e < kV; ++e) {
        if (e0 + e < t1 && (x[u][e] > bv || bi == 0x7fffffff)) {
          bv = x[u][e];
          bi = static_cast<int>(e0 + e);
        }
      }
    }
#pragma unroll
    for (int off = kWave / 2; off >= 1; off /= 2) {
      const float vo = __shfl_xor(bv, off);
      const int io = __shfl_xor(bi, off);
      merge_arg(bv, bi, vo, io);
    }
    if (lane == 0) {
      sh_mx[wave] = bv;
      sh_mi[wave] = bi;
    }
    __syncthreads();
    if (tid == 0) {
      float v = sh_mx[0];
      int ix = sh_mi[0];
      for (int w = 1; w < kWaves; ++w) merge_arg(v, ix, sh_mx[w], sh_mi[w]);
      Partial pr;
      pr.s = 0.0;
      pr.mx = v;
      pr.mi = ix;
      part[tile] = pr;
    }
  }
}

// ================================================================== K2
constexpr int kK2Block = 128;  // covers the 2*SV_GAMMA_MAX+1 rows of a request

template <int DT>
__global__ __launch_bounds__(kK2Block) void k2_decide(
    const void *__restrict__ target, const void *__restrict__ draft,
    const int32_t *__restrict__ tokens, const float *__restrict__ u_accept,
    const float *__restrict__ temps, float scalar_T, const int32_t *__restrict__ lens, int gamma,
    int V, int NS, const Partial *__restrict__ part, int32_t *__restrict__ accepted_count,
    int32_t *__restrict__ out_tokens, SelParams *__restrict__ sel, unsigned *__restrict__ counters,
    sv_debug dbg) {
  const int b = blockIdx.x;
  const int tid = threadIdx.x;
  const int rows = 2 * gamma + 1;
  const int g = request_len(lens, gamma, b);
  const float T = request_T(temps, scalar_T, b);
  const bool greedy = !(T > 0.0f);
  const float c = greedy ? 0.0f : temp_scale(T);

  __shared__ double sh_L[2 * SV_GAMMA_MAX + 1];   // log2 of the row's partition sum
  __shared__ double sh_s[2 * SV_GAMMA_MAX + 1];
  __shared__ int sh_M[2 * SV_GAMMA_MAX + 1];
  __shared__ int sh_arg[2 * SV_GAMMA_MAX + 1];
  __shared__ int sh_k;

  // merge the tile partials of each needed row, tiles in increasing order
  if (tid < rows) {
    const int r = tid;
    const bool is_target = r <= gamma;
    const int i = is_target ? r : r - gamma - 1;
    const bool needed = is_target ? (i <= g) : (!greedy && i < g);
    if (needed) {
      const Partial *pp = part + (static_cast<long>(b) * rows + r) * NS;
      if (!greedy) {
        int M = pp[0].mi;
        double s = pp[0].s;
        float mx = pp[0].mx;
        for (int jj = 1; jj < NS; ++jj) merge_sm(M, s, mx, pp[jj].mi, pp[jj].s, pp[jj].mx);
        sh_M[r] = M;
        sh_s[r] = s;
        sh_L[r] = static_cast<double>(M) + log2(s);
        if (dbg.row_max) dbg.row_max[static_cast<long>(b) * rows + r] = mx;
        if (dbg.row_sum)  // sum_v exp((z_v - max)/T) = s * 2^(M - max c)
          dbg.row_sum[static_cast<long>(b) * rows + r] =
              s * exp2(static_cast<double>(M) - static_cast<double>(mx) * static_cast<double>(c));
      } else {
        float v = pp[0].mx;
        int ix = pp[0].mi;
        for (int jj = 1; jj < NS; ++jj) merge_arg(v, ix, pp[jj].mx, pp[jj].mi);
        sh_arg[r] = ix;
        if (dbg.row_argmax && is_target) dbg.row_argmax[static_cast<long>(b) * (gamma + 1) + r] = ix;
      }
    }
  }
  __syncthreads();

  // acceptance of each draft and the first rejection (one wave, gamma <= 32)
  if (tid < kWave) {
    bool reject = false;
    if (tid < g) {
      const int x = tokens[static_cast<long>(b) * gamma + tid];
      if (x < 0 || x >= V) {
        reject = true;  // a draft id outside the vocabulary is rejected, never dereferenced
      } else if (greedy) {
        reject = (x != sh_arg[tid]);
      } else {
        const char *trow = static_cast<const char *>(target) +
                           (static_cast<long>(b) * (gamma + 1) + tid) * V * Elem<DT>::kBytes;
        const char *drow = static_cast<const char *>(draft) +
                           (static_cast<long>(b) * gamma + tid) * V * Elem<DT>::kBytes;
        const double cd = static_cast<double>(c);
        // log2 p_i(x) and log2 q_i(x) in fp64: z*c - log2(sum 2^(z c))
        const double lp = static_cast<double>(load_one<DT>(trow, x)) * cd - sh_L[tid];
        const double lq = static_cast<double>(load_one<DT>(drow, x)) * cd - sh_L[gamma + 1 + tid];
        const double ratio = exp2(lp - lq);
        const double a = ratio < 1.0 ? ratio : 1.0;
        reject = !(static_cast<double>(u_accept[static_cast<long>(b) * gamma + tid]) < a);
        const long o = static_cast<long>(b) * gamma + tid;
        if (dbg.p_draft) dbg.p_draft[o] = exp2(lp);
        if (dbg.q_draft) dbg.q_draft[o] = exp2(lq);
        if (dbg.accept_prob) dbg.accept_prob[o] = a;
      }
    }
    const unsigned long long rej = __ballot(reject);
    if (tid == 0) sh_k = rej ? (__ffsll(static_cast<long long>(rej)) - 1) : g;
  }
  __syncthreads();
  const int k = sh_k;

  // accepted prefix, the greedy replacement / bonus, -1 padding
  for (int t = tid; t <= gamma; t += kK2Block) {
    int32_t v = -1;
    if (t < k) v = tokens[static_cast<long>(b) * gamma + t];
    else if (t == k && greedy) v = sh_arg[k];
    out_tokens[static_cast<long>(b) * (gamma + 1) + t] = v;
  }
  if (tid == 0) {
    accepted_count[b] = k;
    SelParams sp;
    sp.k = k;
    sp.c = c;
    if (greedy) {
      sp.mode = 0;
      sp.negMp = sp.negMq = 0.0f;
      sp.r = 0.0f;
      sp.ip = 0.0;
    } else {
      sp.mode = (k < g) ? 1 : 2;
      sp.negMp = -static_cast<float>(sh_M[k]);
      sp.ip = 1.0 / sh_s[k];
      if (k < g) {
        sp.negMq = -static_cast<float>(sh_M[gamma + 1 + k]);
        sp.r = static_cast<float>(sh_s[k] / sh_s[gamma + 1 + k]);
      } else {
        sp.negMq = 0.0f;
        sp.r = 0.0f;
      }
    }
    sel[b] = sp;
    counters[b] = 0u;
  }
}

// ================================================================== K3
// w(v) in units of the target row's scale s'_p:  p(v) - q(v) = (e_p - e_q r) / s'_p
// with e_p = 2^(z_p c - M_p), e_q = 2^(z_q c - M_q), r = s'_p / s'_q.  A common
// scale does not move the normalised CDF, so sampling never divides by s'_p.
template <int DT>
__device__ __forceinline__ void residual_lane(const SelParams &sp, const void *trow,
                                              const void *drow, bool aligned, long e0, long V,
                                              float *w, float *p) {
  float zp[8], zq[8];
  if constexpr (DT == SV_BF16) {
    load_vec_guarded<DT>(trow, aligned, e0, V, zp);
    if (sp.mode == 1) load_vec_guarded<DT>(drow, aligned, e0, V, zq);
  } else {
    load_vec_guarded<DT>(trow, aligned, e0, V, zp);
    load_vec_guarded<DT>(trow, aligned, e0 + 4, V, zp + 4);
    if (sp.mode == 1) {
      load_vec_guarded<DT>(drow, aligned, e0, V, zq);
      load_vec_guarded<DT>(drow, aligned, e0 + 4, V, zq + 4);
    }
  }
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    const float ep = __builtin_amdgcn_exp2f(fmaf(zp[e], sp.c, sp.negMp));  // -inf -> 0
    p[e] = ep;
    if (sp.mode == 1) {
      const float eq = __builtin_amdgcn_exp2f(fmaf(zq[e], sp.c, sp.negMq));
      w[e] = fmaxf(0.0f, fmaf(-eq, sp.r, ep));
    } else {
      w[e] = ep;
    }
  }
}

__device__ __forceinline__ float sum8(const float *a) {
  return ((a[0] + a[1]) + (a[2] + a[3])) + ((a[4] + a[5]) + (a[6] + a[7]));
}

__device__ __forceinline__ double wave_sum(double v) {
#pragma unroll
  for (int off = kWave / 2; off >= 1; off /= 2) v += __shfl_xor(v, off);
  return v;
}

// inclusive prefix over the 64 lanes of a wave (fp64)
__device__ __forceinline__ double wave_scan(double v, int lane) {
#pragma unroll
  for (int off = 1; off < kWave; off *= 2) {
    const double o = __shfl_up(v, off);
    if (lane >= off) v += o;
  }
  return v;
}

// inclusive prefix over the 256 threads of a workgroup (fp64); returns the total in *total
__device__ __forceinline__ double block_scan(double v, double *sh, double *total) {
  const int tid = threadIdx.x, lane = tid & (kWave - 1), wave = tid / kWave;
  v = wave_scan(v, lane);
  if (lane == kWave - 1) sh[wave] = v;
  __syncthreads();
  double before = 0.0;
  for (int w = 0; w < wave; ++w) before += sh[w];
  double tot = 0.0;
  for (int w = 0; w < kWaves; ++w) tot += sh[w];
  __syncthreads();
  *total = tot;
  return v + before;
}

template <int DT>
__global__ __launch_bounds__(kBlock) void k3_sample(
    const void *__restrict__ target, const void *__restrict__ draft,
    const float *__restrict__ u_sample, int gamma, int V, int NSUB, int SPW, int NW,
    const SelParams *__restrict__ sel, SubSums *__restrict__ sums, unsigned *__restrict__ counters,
    int32_t *__restrict__ out_tokens, double *__restrict__ dbg_mass) {
  const int b = blockIdx.x / NW;
  const int wg = blockIdx.x % NW;
  const SelParams sp = sel[b];
  if (sp.mode == 0) return;
  const int tid = threadIdx.x, lane = tid & (kWave - 1), wave = tid / kWave;
  const void *trow = static_cast<const char *>(target) +
                     (static_cast<long>(b) * (gamma + 1) + sp.k) * V * Elem<DT>::kBytes;
  const void *drow = (sp.mode == 1)
                         ? static_cast<const void *>(static_cast<const char *>(draft) +
                                                     (static_cast<long>(b) * gamma + sp.k) * V *
                                                         Elem<DT>::kBytes)
                         : nullptr;
  const bool aligned = ((reinterpret_cast<uintptr_t>(trow) | reinterpret_cast<uintptr_t>(drow)) & 15u) == 0;
  SubSums *bs = sums + static_cast<long>(b) * NSUB;

  // pass 1: the mass of each 512-token sub-chunk this workgroup owns
  for (int t = 0; t < SPW; ++t) {
    const int s = (wg * kWaves + wave) * SPW + t;
    if (s >= NSUB) break;
    float w[8], p[8];
    residual_lane<DT>(sp, trow, drow, aligned, static_cast<long>(s) * kSub + lane * 8, V, w, p);
    const double sw = wave_sum(static_cast<double>(sum8(w)));
    const double spp = wave_sum(static_cast<double>(sum8(p)));
    if (lane == 0) {
      SubSums ss;
      ss.w = sw;
      ss.p = spp;
      bs[s] = ss;
      __threadfence();  // release the sums before the arrival count
    }
  }
  __shared__ int sh_last;
  __syncthreads();
  if (tid == 0) {
    __threadfence();
    const unsigned prev = atomicAdd(&counters[b], 1u);
    sh_last = (prev == static_cast<unsigned>(NW - 1));
  }
  __syncthreads();
  if (!sh_last) return;
  __threadfence();  // acquire: every workgroup's sums are visible

  // pass 2 (last workgroup): total mass, then the sub-chunk holding u*Z
  __shared__ double sh_scan[kWaves];
  __shared__ int sh_sub;
  __shared__ double sh_base;
  double Zw = 0.0, Zp = 0.0;
  for (int base = 0; base < NSUB; base += kBlock) {
    const int s = base + tid;
    double tw, tp;
    block_scan((s < NSUB) ? bs[s].w : 0.0, sh_scan, &tw);
    block_scan((s < NSUB) ? bs[s].p : 0.0, sh_scan, &tp);
    Zw += tw;
    Zp += tp;
  }
  const bool use_p = !(Zw > 0.0);  // zero residual mass: fall back to p_k
  const double Z = use_p ? Zp : Zw;
  const double target_mass = static_cast<double>(u_sample[b]) * Z;
  if (tid == 0) sh_sub = 0x7fffffff;
  __syncthreads();
  double run = 0.0;
  for (int base = 0; base < NSUB; base += kBlock) {
    const int s = base + tid;
    const double v = (s < NSUB) ? (use_p ? bs[s].p : bs[s].w) : 0.0;
    double tot;
    const double incl = block_scan(v, sh_scan, &tot);
    // lowest sub-chunk with mass whose inclusive prefix exceeds u*Z
    if (s < NSUB && v > 0.0 && run + incl > target_mass) atomicMin(&sh_sub, s);
    __syncthreads();
    if (s == sh_sub) sh_base = run + (incl - v);
    __syncthreads();
    if (sh_sub != 0x7fffffff) break;
    run += tot;
  }
  if (sh_sub == 0x7fffffff) {  // rounding left u*Z at the very end: last sub-chunk with mass
    __syncthreads();
    if (tid == 0) {
      int last = NSUB - 1;
      for (int s = NSUB - 1; s >= 0; --s) {
        if ((use_p ? bs[s].p : bs[s].w) > 0.0) {
          last = s;
          break;
        }
      }
      double acc = 0.0;
      for (int s = 0; s < last; ++s) acc += use_p ? bs[s].p : bs[s].w;
      sh_sub = last;
      sh_base = acc;
    }
    __syncthreads();
  }
  const int sub = sh_sub;
  const double base_mass = sh_base;

  // pass 3 (wave 0 of the last workgroup): the token inside the sub-chunk.  Each
  // lane proposes its first token with mass whose running prefix exceeds u*Z;
  // the lowest proposing lane wins.  Tokens with zero mass are never chosen.
  if (wave == 0) {
    float w[8], p[8];
    const long e0 = static_cast<long>(sub) * kSub + lane * 8;
    residual_lane<DT>(sp, trow, drow, aligned, e0, V, w, p);
    const float *vals = use_p ? p : w;
    const double lsum = static_cast<double>(sum8(vals));
    const double incl = wave_scan(lsum, lane);
    double acc = base_mass + (incl - lsum);
    int cand = -1, last_pos = -1;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      if (vals[e] > 0.0f) {
        last_pos = e;
        acc += static_cast<double>(vals[e]);
        if (cand < 0 && target_mass < acc) cand = e;
      }
    }
    const unsigned long long props = __ballot(cand >= 0);
    const long dst = static_cast<long>(b) * (gamma + 1) + sp.k;
    if (props) {
      const int L = __ffsll(static_cast<long long>(props)) - 1;
      if (lane == L) out_tokens[dst] = static_cast<int>(e0 + cand);
    } else {
      // rounding left u*Z past the sub-chunk: its last token with mass
      const unsigned long long has = __ballot(last_pos >= 0);
      const int L = has ? 63 - __clzll(static_cast<long long>(has)) : 0;
      if (lane == L) out_tokens[dst] = static_cast<int>(e0 + (last_pos >= 0 ? last_pos : 0));
    }
    if (lane == 0 && dbg_mass) dbg_mass[b] = Z * sp.ip;
  }
}

// ================================================================== host side
struct Plan {
  int rows, U, NS, NSUB, SPW, NW;
  long k1_tiles, k3_groups;
  size_t part_off, sel_off, sums_off, cnt_off, total;
};

size_t align_up(size_t x) { return (x + kAlign - 1) / kAlign * kAlign; }

bool make_plan(int B, int gamma, int V, int dtype, Plan *P) {
  if (B < 1 || gamma < 0 || gamma > SV_GAMMA_MAX || V < 1) return false;
  if (dtype != SV_F32 && dtype != SV_BF16) return false;
  const int vec = dtype == SV_BF16 ? 8 : 4;
  P->rows = 2 * gamma + 1;
  const long slots = static_cast<long>(B) * P->rows;
  // largest tile (up to 64 elements per thread) that still gives >= 1024 workgroups
  int U = 8;
  while (U > 1 && slots * ((V + static_cast<long>(kBlock) * U * vec - 1) / (static_cast<long>(kBlock) * U * vec)) < 1024)
    U /= 2;
  P->U = U;
  const long tile = static_cast<long>(kBlock) * U * vec;
  P->NS = static_cast<int>((V + tile - 1) / tile);
  P->k1_tiles = slots * P->NS;
  P->NSUB = (V + kSub - 1) / kSub;
  int SPW = 4;
  while (SPW > 1 && static_cast<long>(B) * ((P->NSUB + kWaves * SPW - 1) / (kWaves * SPW)) < 1024) SPW /= 2;
  P->SPW = SPW;
  P->NW = (P->NSUB + kWaves * SPW - 1) / (kWaves * SPW);
  P->k3_groups = static_cast<long>(B) * P->NW;
  // 1-D grids: work-items per launch must stay below 2^32
  const long max_groups = (1L << 32) / kBlock - 1;
  if (P->k1_tiles > max_groups || P->k3_groups > max_groups) return false;
  size_t off = 0;
  P->part_off = off;
  off = align_up(off + sizeof(Partial) * static_cast<size_t>(P->k1_tiles));
  P->sel_off = off;
  off = align_up(off + sizeof(SelParams) * static_cast<size_t>(B));
  P->sums_off = off;
  off = align_up(off + sizeof(SubSums) * static_cast<size_t>(B) * P->NSUB);
  P->cnt_off = off;
  off = align_up(off + sizeof(unsigned) * static_cast<size_t>(B));
  P->total = off;
  return true;
}

template <int DT>
hipError_t launch_k1(int U, const void *target, const void *draft, const float *temps, float scalar_T,
                     const int32_t *lens, int gamma, int V, const Plan &P, Partial *part,
                     hipStream_t st) {
  dim3 grid(static_cast<unsigned>(P.k1_tiles)), block(kBlock);
  switch (U) {
    case 8: hipLaunchKernelGGL((k1_row_stats<DT, 8>), grid, block, 0, st, target, draft, temps, scalar_T, lens, gamma, V, P.NS, part); break;
    case 4: hipLaunchKernelGGL((k1_row_stats<DT, 4>), grid, block, 0, st, target, draft, temps, scalar_T, lens, gamma, V, P.NS, part); break;
    case 2: hipLaunchKernelGGL((k1_row_stats<DT, 2>), grid, block, 0, st, target, draft, temps, scalar_T, lens, gamma, V, P.NS, part); break;
    default: hipLaunchKernelGGL((k1_row_stats<DT, 1>), grid, block, 0, st, target, draft, temps, scalar_T, lens, gamma, V, P.NS, part); break;
  }
  return hipGetLastError();
}

template <int DT>
int run(const void *target, const void *draft, const int32_t *tokens, const float *u_accept,
        const float *u_sample, const float *temps, float scalar_T, bool all_greedy,
        const int32_t *lens, int B, int gamma, int V, int32_t *count, int32_t *out, void *ws,
        const Plan &P, hipStream_t st, const sv_debug *dbgp) {
  char *base = static_cast<char *>(ws);
  Partial *part = reinterpret_cast<Partial *>(base + P.part_off);
  SelParams *sel = reinterpret_cast<SelParams *>(base + P.sel_off);
  SubSums *sums = reinterpret_cast<SubSums *>(base + P.sums_off);
  unsigned *cnt = reinterpret_cast<unsigned *>(base + P.cnt_off);
  sv_debug dbg;
  memset(&dbg, 0, sizeof dbg);
  if (dbgp) dbg = *dbgp;
  const bool timed = dbg.k1_events[0] && dbg.k1_events[1];
  if (timed && hipEventRecord(static_cast<hipEvent_t>(dbg.k1_events[0]), st) != hipSuccess) return SV_EHIP;
  hipError_t e = launch_k1<DT>(P.U, target, draft, temps, scalar_T, lens, gamma, V, P, part, st);
  if (e != hipSuccess) return SV_EHIP;
  if (timed && hipEventRecord(static_cast<hipEvent_t>(dbg.k1_events[1]), st) != hipSuccess) return SV_EHIP;
  hipLaunchKernelGGL((k2_decide<DT>), dim3(B), dim3(kK2Block), 0, st, target, draft, tokens, u_accept,
                     temps, scalar_T, lens, gamma, V, P.NS, part, count, out, sel, cnt, dbg);
  if (hipGetLastError() != hipSuccess) return SV_EHIP;
  if (!all_greedy) {
    hipLaunchKernelGGL((k3_sample<DT>), dim3(static_cast<unsigned>(P.k3_groups)), dim3(kBlock), 0, st,
                       target, draft, u_sample, gamma, V, P.NSUB, P.SPW, P.NW, sel, sums, cnt, out,
                       dbg.residual_mass);
    if (hipGetLastError() != hipSuccess) return SV_EHIP;
  }
  return SV_OK;
}

int dispatch(const void *target, const void *draft, const int32_t *tokens, const float *u_accept,
             const float *u_sample, const float *temps, float scalar_T, bool all_greedy,
             const int32_t *lens, int B, int gamma, int V, int dtype, int32_t *count, int32_t *out,
             void *ws, size_t ws_bytes, void *stream, const sv_debug *dbg) {
  Plan P;
  if (!make_plan(B, gamma, V, dtype, &P)) return SV_EINVAL;
  if (!target || !u_sample || !count || !out) return SV_EINVAL;
  if (gamma > 0 && !tokens) return SV_EINVAL;
  if (gamma > 0 && !all_greedy && (!draft || !u_accept)) return SV_EINVAL;
  if (!ws || (reinterpret_cast<uintptr_t>(ws) % kAlign) != 0 || ws_bytes < P.total) return SV_EWORKSPACE;
  if (dbg && ((dbg->k1_events[0] == nullptr) != (dbg->k1_events[1] == nullptr))) return SV_EINVAL;
  hipStream_t st = static_cast<hipStream_t>(stream);
  if (dtype == SV_BF16)
    return run<SV_BF16>(target, draft, tokens, u_accept, u_sample, temps, scalar_T, all_greedy, lens, B,
                        gamma, V, count, out, ws, P, st, dbg);
  return run<SV_F32>(target, draft, tokens, u_accept, u_sample, temps, scalar_T, all_greedy, lens, B,
                     gamma, V, count, out, ws, P, st, dbg);
}

}  // namespace

// ================================================================== C ABI
extern "C" {

size_t spec_verify_workspace_bytes(int B, int gamma, int V, int dtype) {
  Plan P;
  if (!make_plan(B, gamma, V, dtype, &P)) return 0;
  return P.total;
}

int spec_verify(const void *target_logits, const void *draft_logits, const int32_t *draft_tokens,
                const float *u_accept, const float *u_sample, float temperature, int B, int gamma,
                int V, int dtype, int32_t *accepted_count, int32_t *out_tokens, void *workspace,
                size_t workspace_bytes, void *stream) {
  if (!(temperature >= 0.0f) || isinf(temperature)) return SV_EINVAL;
  return dispatch(target_logits, draft_logits, draft_tokens, u_accept, u_sample, nullptr, temperature,
                  temperature == 0.0f, nullptr, B, gamma, V, dtype, accepted_count, out_tokens,
                  workspace, workspace_bytes, stream, nullptr);
}

int spec_verify_ex(const void *target_logits, const void *draft_logits, const int32_t *draft_tokens,
                   const float *u_accept, const float *u_sample, const float *temperature,
                   const int32_t *draft_lens, int B, int gamma, int V, int dtype,
                   int32_t *accepted_count, int32_t *out_tokens, void *workspace,
                   size_t workspace_bytes, void *stream, const sv_debug *dbg) {
  if (!temperature) return SV_EINVAL;
  return dispatch(target_logits, draft_logits, draft_tokens, u_accept, u_sample, temperature, 0.0f,
                  false, draft_lens, B, gamma, V, dtype, accepted_count, out_tokens, workspace,
                  workspace_bytes, stream, dbg);
}

const char *spec_verify_strerror(int code) {
  switch (code) {
    case SV_OK: return "success";
    case SV_EINVAL: return "invalid argument (pointer, size, dtype or temperature)";
    case SV_EWORKSPACE: return "workspace missing, not 256-byte aligned, or too small";
    case SV_EHIP: return "HIP launch or runtime call failed";
    default: return "unknown error code";
  }
}

}  // extern "C"
