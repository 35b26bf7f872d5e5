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
// Two launches on the caller's stream for the verify step (three when a row has
// more than 512 sub-chunks), no host synchronisation, no device-wide fences:
// K1's results reach K2 through the kernel boundary, and K2's workgroups hand
// their sub-chunk masses to each other through device-scope atomic words.
//
//   K1  k1_row_stats    one workgroup per (request, logit row, vocabulary chunk).
//                       Streams the chunk once (16-byte non-temporal loads, next
//                       tile prefetched) and produces, for a stochastic row,
//                       (M, s) with M an integer upper bound of max(z)*log2(e)/T
//                       and s = sum 2^(z*c - M); for a greedy row, the maximum
//                       and its lowest index.  Integer M makes every rescale
//                       between partial sums an exact power of two (ldexp).
//   K2  k2_decide_mass  NW workgroups per request.  Each merges the chunk
//                       partials of every row in a fixed order, evaluates
//                       a_i = min(1, p_i(x_i)/q_i(x_i)) in fp64 from the two
//                       gathered logits and finds the first rejection with a
//                       wave ballot (workgroup 0 stores the outputs); then its
//                       waves write the mass of w = max(0, p - q) (or p for the
//                       bonus) of the selected row pair per 2048-token sub-chunk;
//                       then the sub-chunk whose prefix crosses u*Z, and the
//                       token inside it, are found by the workgroup that
//                       computed that sub-chunk (or by workgroup 0).
//   K3  k3_select       the same draw as a kernel of its own, one workgroup per
//                       request, for rows of more than 512 sub-chunks.
//   KS  k_small_verify  one 1024-thread workgroup per request, the whole step in
//                       one launch, when a request's rows hold at most 12288
//                       logits: the rows are staged in LDS with one batch of
//                       loads, and the statistics, decision and draw follow on
//                       chip.
//
// Extensions, on the same row statistics:
//   top-k / top-p       k_filter_capture, k_filter_deep_count, k_filter_resolve
//                       and k_filter_general between K1 and K2 find each
//                       filtered row's cut; K2 and K3 are instantiated with
//                       the cut compares.
//   tree of drafts      K1 over every tree position, then k_tree_walk (a team
//                       of workgroups per request).
//   draft-side sampling k_sample_stats (several workgroups per row), then
//                       k_sample_pick (one wave per row).
//
// Numerics: bf16 -> fp32 widening is exact; exponentials are v_exp_f32 of
// fma(z, c, -M); per-thread partial sums are fp32 over at most 64 terms and
// everything above a thread (wave, workgroup, tile, CDF prefix) is fp64.
#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>

#include <limits.h>
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#include <mutex>

#include "specverify.h"

namespace {

constexpr int kBlock = 256;          // threads per workgroup (4 waves of 64)
constexpr int kWave = 64;
constexpr int kWaves = kBlock / kWave;
constexpr int kSub = 2048;           // tokens per K3 sub-chunk (64 lanes x 32)
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

// Element e of a row as raw bits (bf16: zero-extended), and their value.
template <int DT>
__device__ __forceinline__ unsigned load_bits(const void *row, long e) {
  if constexpr (DT == SV_F32) return static_cast<const unsigned *>(row)[e];
  else return static_cast<unsigned>(static_cast<const uint16_t *>(row)[e]);
}
template <int DT>
__device__ __forceinline__ float bits_value(unsigned v) {
  return __uint_as_float(DT == SV_F32 ? v : v << 16);
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
  float tau_p;   // target row k keeps z >= tau_p (-inf: no filter)
  float tau_q;   // draft row k keeps z >= tau_q
};

struct alignas(16) SubSums {
  double w;  // sum of w over the sub-chunk (target-row units)
  double p;  // sum of 2^(z_p c - M_p) over the sub-chunk (zero-mass fallback)
};

// ------------------------------------------------------------------ hand-over between workgroups
// Where workgroups of one kernel read each other's results (the tree walk's
// shared passes), the values go through device-scope atomic stores and loads:
// each XCD has its own L2, not coherent with the others, and these accesses
// bypass it, so no cache write-back or invalidate is needed (a device-scope
// fence would write back or invalidate the XCD's whole L2).  Each value travels
// in one 64-bit word together with a tag the reader waits for, so no store
// completion or counter needs to be awaited.
template <bool COH, typename T>
__device__ __forceinline__ void put(T *p, T v) {
  if constexpr (COH) __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  else *p = v;
}
template <bool COH, typename T>
__device__ __forceinline__ T get(const T *p) {
  if constexpr (COH) return __hip_atomic_load(const_cast<T *>(p), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  else return *p;
}

constexpr unsigned kSpinLimit = 1u << 20;  // polls of a bounded wait (about a second; a correct run needs a few)

// ------------------------------------------------------------------ wave reductions
// fp64 wave scan / sum with DPP row shifts and row broadcasts (no LDS round
// trip).  Lanes without a source read 0, the identity of the sum.  Called with
// the whole wave active.
template <int CTRL, int ROW_MASK>
__device__ __forceinline__ double dpp_f64(double x) {
  const long long bits = __double_as_longlong(x);
  const int lo = __builtin_amdgcn_update_dpp(0, static_cast<int>(bits), CTRL, ROW_MASK, 0xf, true);
  const int hi = __builtin_amdgcn_update_dpp(0, static_cast<int>(bits >> 32), CTRL, ROW_MASK, 0xf, true);
  return __longlong_as_double((static_cast<long long>(hi) << 32) | static_cast<unsigned>(lo));
}

// inclusive prefix over the 64 lanes of a wave
__device__ __forceinline__ double wave_scan(double v, int /*lane*/) {
  v += dpp_f64<0x111, 0xf>(v);  // row_shr:1
  v += dpp_f64<0x112, 0xf>(v);  // row_shr:2
  v += dpp_f64<0x114, 0xf>(v);  // row_shr:4
  v += dpp_f64<0x118, 0xf>(v);  // row_shr:8   (each row of 16 now holds its own prefix)
  v += dpp_f64<0x142, 0xa>(v);  // row_bcast:15 into rows 1 and 3
  v += dpp_f64<0x143, 0xc>(v);  // row_bcast:31 into rows 2 and 3
  return v;
}

__device__ __forceinline__ double lane_value(double v, int lane) {
  const long long bits = __double_as_longlong(v);
  const int lo = __builtin_amdgcn_readlane(static_cast<int>(bits), lane);
  const int hi = __builtin_amdgcn_readlane(static_cast<int>(bits >> 32), lane);
  return __longlong_as_double((static_cast<long long>(hi) << 32) | static_cast<unsigned>(lo));
}

// sum over the wave, the same value in every lane
__device__ __forceinline__ double wave_sum(double v) { return lane_value(wave_scan(v, 0), kWave - 1); }

// maximum over the wave, the same value in every lane (lanes without a DPP
// source keep -inf, the identity)
__device__ __forceinline__ float wave_max_f32(float v) {
  v = fmaxf(v, __int_as_float(__builtin_amdgcn_update_dpp(__float_as_int(-INFINITY), __float_as_int(v), 0x111, 0xf, 0xf, false)));
  v = fmaxf(v, __int_as_float(__builtin_amdgcn_update_dpp(__float_as_int(-INFINITY), __float_as_int(v), 0x112, 0xf, 0xf, false)));
  v = fmaxf(v, __int_as_float(__builtin_amdgcn_update_dpp(__float_as_int(-INFINITY), __float_as_int(v), 0x114, 0xf, 0xf, false)));
  v = fmaxf(v, __int_as_float(__builtin_amdgcn_update_dpp(__float_as_int(-INFINITY), __float_as_int(v), 0x118, 0xf, 0xf, false)));
  v = fmaxf(v, __int_as_float(__builtin_amdgcn_update_dpp(__float_as_int(-INFINITY), __float_as_int(v), 0x142, 0xa, 0xf, false)));
  v = fmaxf(v, __int_as_float(__builtin_amdgcn_update_dpp(__float_as_int(-INFINITY), __float_as_int(v), 0x143, 0xc, 0xf, false)));
  return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), kWave - 1));
}

// integer maximum / minimum over the wave, the same value in every lane
template <bool MAX>
__device__ __forceinline__ int wave_ext_i32(int v) {
  constexpr int id = MAX ? INT_MIN : INT_MAX;
  auto f = [](int x, int y) { return MAX ? (x > y ? x : y) : (x < y ? x : y); };
  v = f(v, __builtin_amdgcn_update_dpp(id, v, 0x111, 0xf, 0xf, false));
  v = f(v, __builtin_amdgcn_update_dpp(id, v, 0x112, 0xf, 0xf, false));
  v = f(v, __builtin_amdgcn_update_dpp(id, v, 0x114, 0xf, 0xf, false));
  v = f(v, __builtin_amdgcn_update_dpp(id, v, 0x118, 0xf, 0xf, false));
  v = f(v, __builtin_amdgcn_update_dpp(id, v, 0x142, 0xa, 0xf, false));
  v = f(v, __builtin_amdgcn_update_dpp(id, v, 0x143, 0xc, 0xf, false));
  return __builtin_amdgcn_readlane(v, kWave - 1);
}

// ================================================================== K1
// Rows of request b: r in [0, gamma] are target rows, r in [gamma+1, 2 gamma]
// are draft rows r - gamma - 1.  A row is needed if it is a target row i <= g_b,
// or a draft row i < g_b of a stochastic request (greedy requests never read
// draft logits).
//
// Workgroup w handles chunk j = w % NCH of row slot w / NCH.  A chunk is a run
// of 16-byte vectors [v0, v1) streamed in tiles of U vectors per thread; the
// next tile's loads are issued before the current tile is reduced, and loads
// are non-temporal (each logit is read once here).  Elements that do not fill
// a whole aligned vector (the row tail, or every element of a row that is not
// 16-byte aligned) are read one by one by the row's last chunk / by all chunks.
typedef unsigned u32x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ u32x4 load_nt(const u32x4 *p) { return __builtin_nontemporal_load(p); }

template <int DT>
__device__ __forceinline__ void widen_vec(u32x4 v, float *x) {
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

// -inf in every element of a vector (neutral for max and for sums of exponentials)
template <int DT>
__device__ __forceinline__ u32x4 neg_inf_vec() {
  if constexpr (DT == SV_F32) return u32x4{0xff800000u, 0xff800000u, 0xff800000u, 0xff800000u};
  return u32x4{0xff80ff80u, 0xff80ff80u, 0xff80ff80u, 0xff80ff80u};
}

// Tile statistics folded into a thread's running (M, s, max): M_t = ceil(max*c)
// makes every term 2^(z*c - M_t) <= 1 (up to one rounding), and the fold
// rescales by an exact power of two.
template <int N>
__device__ __forceinline__ void fold_values(const float *x, float c, int &M, double &s, float &mx) {
  float tmx = -INFINITY;
#pragma unroll
  for (int e = 0; e < N; ++e) tmx = fmaxf(tmx, x[e]);
  if (tmx > -INFINITY) {
    const float Mf = ceilf(tmx * c);
    float acc = 0.0f;
#pragma unroll
    for (int e = 0; e < N; ++e) acc += __builtin_amdgcn_exp2f(fmaf(x[e], c, -Mf));
    merge_sm(M, s, mx, static_cast<int>(Mf), static_cast<double>(acc), tmx);
  }
}

// The same for a tile held as U raw 16-byte vectors, widened once for the
// maximum and again for the sum (the compiler may keep the first widening in
// registers instead of repeating it).
template <int DT, int U>
__device__ __forceinline__ void fold_tile(const u32x4 *v, float c, int &M, double &s, float &mx) {
  constexpr int kV = Elem<DT>::kVec;
  float tmx = -INFINITY;
#pragma unroll
  for (int u = 0; u < U; ++u) {
    float x[kV];
    widen_vec<DT>(v[u], x);
#pragma unroll
    for (int e = 0; e < kV; ++e) tmx = fmaxf(tmx, x[e]);
  }
  if (tmx > -INFINITY) {
    const float Mf = ceilf(tmx * c);
    const float nM = -Mf;
    static_assert(U * kV >= 8, "a tile fills the eight accumulators");
    float acc[8];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      float x[kV];
      widen_vec<DT>(v[u], x);
#pragma unroll
      for (int e = 0; e < kV; ++e) {
        // the first eight terms start the accumulators (no add of zero)
        const int i = u * kV + e;
        const float t = __builtin_amdgcn_exp2f(fmaf(x[e], c, nM));
        if (i < 8)
          acc[i] = t;
        else
          acc[i & 7] += t;
      }
    }
    const float ts = ((acc[0] + acc[1]) + (acc[2] + acc[3])) + ((acc[4] + acc[5]) + (acc[6] + acc[7]));
    merge_sm(M, s, mx, static_cast<int>(Mf), static_cast<double>(ts), tmx);
  }
}

// U vectors per thread of the tile starting at vector t0 of the chunk [.., v1).
// Every lane loads (indices are clamped into the chunk, so the code is straight
// line and the compiler can wait for exactly the older tile); with MASK, lanes
// past v1 then hold -inf, else they hold a copy of the chunk's last vector and
// the fold masks them itself (mask_tile).
template <int DT, int U, int BS = kBlock, bool MASK = true>
__device__ __forceinline__ void load_tile(const u32x4 *rv, int t0, int v1, int tid, u32x4 *dst) {
#pragma unroll
  for (int u = 0; u < U; ++u) {
    const int vi = t0 + u * BS + tid;
    const u32x4 x = load_nt(rv + min(vi, v1 - 1));
    dst[u] = (!MASK || vi < v1) ? x : neg_inf_vec<DT>();
  }
}

// The vectors of a tile loaded without MASK, those past v1 replaced by -inf.
template <int DT, int U, int BS = kBlock>
__device__ __forceinline__ void mask_tile(const u32x4 *src, int t0, int v1, int tid, u32x4 *dst) {
#pragma unroll
  for (int u = 0; u < U; ++u) dst[u] = (t0 + u * BS + tid < v1) ? src[u] : neg_inf_vec<DT>();
}

// Streams the vectors [v0, v1) of a row in tiles of U vectors per thread with
// two register buffers: the next tile is in flight while the current one is
// folded.  fold(tile, t0) sees each tile once, in order.  With PRE the first
// tile has already been loaded (load_tile with the same MASK) into `pre`.
template <int DT, int U, int BS, bool MASK, bool PRE, typename Fold>
__device__ __forceinline__ void stream_chunk_impl(const u32x4 *rv, int v0, int v1, int tid, const u32x4 *pre,
                                                  Fold &&fold) {
  constexpr int kTileVecs = U * BS;
  if (v0 >= v1) return;
  u32x4 a[U], b[U];
  if constexpr (PRE) {
#pragma unroll
    for (int u = 0; u < U; ++u) a[u] = pre[u];
  } else {
    load_tile<DT, U, BS, MASK>(rv, v0, v1, tid, a);
  }
  for (int t0 = v0;;) {
    load_tile<DT, U, BS, MASK>(rv, t0 + kTileVecs, v1, tid, b);
    fold(a, t0);
    t0 += kTileVecs;
    if (t0 >= v1) break;
    load_tile<DT, U, BS, MASK>(rv, t0 + kTileVecs, v1, tid, a);
    fold(b, t0);
    t0 += kTileVecs;
    if (t0 >= v1) break;
  }
}

template <int DT, int U, int BS = kBlock, bool MASK = true, typename Fold>
__device__ __forceinline__ void stream_chunk(const u32x4 *rv, int v0, int v1, int tid, Fold &&fold) {
  stream_chunk_impl<DT, U, BS, MASK, false>(rv, v0, v1, tid, nullptr, fold);
}

// K1's streaming: unmasked tiles (its folds mask the last one themselves);
// with PRE the first tile is already in `pre`.
template <int DT, int U, bool PRE, typename Fold>
__device__ __forceinline__ void stream_chunk_k1(const u32x4 *rv, int v0, int v1, int tid, const u32x4 *pre,
                                                Fold &&fold) {
  stream_chunk_impl<DT, U, kBlock, false, PRE>(rv, v0, v1, tid, pre, fold);
}

// Which request kinds a K1 instantiation handles: the uniform entry point knows
// on the host whether every row is stochastic or every row greedy.
enum { kMixed = 0, kStochasticOnly = 1, kGreedyOnly = 2 };

template <int DT, int U, int KIND>
__global__ __launch_bounds__(kBlock) void k1_row_stats(
    const void *__restrict__ target, const void *__restrict__ draft,
    const int32_t *__restrict__ tokens, const float *__restrict__ temps, float scalar_T,
    const int32_t *__restrict__ lens, int gamma, int V, int NCH, int chunk_vecs, int grid_rows,
    Partial *__restrict__ part, float *__restrict__ zx, unsigned *__restrict__ row_counter,
    unsigned long long *__restrict__ req_words, int req_words_n) {
  constexpr int kV = Elem<DT>::kVec;
  const int rows = 2 * gamma + 1;
  // the grid covers grid_rows rows per request: all 2 gamma + 1, or the gamma + 1
  // target rows when every request is greedy
  const int gslot = blockIdx.x / NCH;
  const int j = blockIdx.x - gslot * NCH;
  const int b = gslot / grid_rows;
  const int r = gslot - b * grid_rows;
  const int slot = b * rows + r;
  const int wgid = slot * NCH + j;
  // a per-row counter of the kernels that follow (filtered calls), cleared here,
  // and per-request words of the tree walk, by the request's first chunk of row 0
  if (row_counter && j == 0 && threadIdx.x == 0) row_counter[slot] = 0u;
  if (req_words && r == 0 && j == 0)
    for (int t = threadIdx.x; t < req_words_n; t += kBlock) req_words[static_cast<long>(b) * req_words_n + t] = 0ull;
  const bool is_target = r <= gamma;
  const int i = is_target ? r : r - gamma - 1;
  const char *row =
      is_target ? static_cast<const char *>(target) +
                      (static_cast<long>(b) * (gamma + 1) + i) * V * Elem<DT>::kBytes
                : static_cast<const char *>(draft) +
                      (static_cast<long>(b) * gamma + i) * V * Elem<DT>::kBytes;
  const bool aligned = (reinterpret_cast<uintptr_t>(row) & 15u) == 0;
  const int nvec = aligned ? V / kV : 0;  // whole aligned vectors of the row
  const int v0 = min(j * chunk_vecs, nvec);
  const int v1 = min(v0 + chunk_vecs, nvec);
  const u32x4 *rv = reinterpret_cast<const u32x4 *>(row);
  const int tid = threadIdx.x;
  // With per-request temperatures and lengths, whether this row is needed (and
  // how) is known only once temps[b] and lens[b] have arrived.  The first tile
  // of a row every request reads (any target row when the lengths are uniform,
  // else target row 0) is requested before them, so that the two latencies
  // overlap; other rows wait for the parameters.  Requested early as well, the
  // draft rows' tiles were read for nothing in about half of the workgroups of
  // a batch with greedy and short requests, and the target rows' past a ragged
  // request's length cost the ragged B = 128 batch 75.0 against 72.0 us per call.
  constexpr bool kPre = KIND == kMixed;
  const bool early = is_target && (lens == nullptr || i == 0);
  u32x4 pre[U];
  if constexpr (kPre) {
    if (early && v0 < v1) load_tile<DT, U, kBlock, false>(rv, v0, v1, tid, pre);
  }
  const int g = request_len(lens, gamma, b);
  const float T = request_T(temps, scalar_T, b);
  const bool greedy = KIND == kGreedyOnly ? true : (KIND == kStochasticOnly ? false : !(T > 0.0f));
  if (is_target ? (i > g) : (greedy || i >= g)) return;
  if constexpr (kPre) {
    if (!early && v0 < v1) load_tile<DT, U, kBlock, false>(rv, v0, v1, tid, pre);
  }

  // elements read one by one: the tail after the last whole vector (last
  // chunk), or this chunk's share of a row that is not 16-byte aligned
  const long se0 = aligned ? (j == NCH - 1 ? static_cast<long>(nvec) * kV : V)
                           : min(static_cast<long>(j) * chunk_vecs * kV, static_cast<long>(V));
  const long se1 = aligned ? V : min(static_cast<long>(j + 1) * chunk_vecs * kV, static_cast<long>(V));
  // the logit at this position's draft token, picked up by the chunk that owns it
  // (stochastic rows i < g only; ids outside [0, V) are never dereferenced)
  if (tid == 0 && !greedy && i < g) {
    const int x = tokens[static_cast<long>(b) * gamma + i];
    if (x >= 0 && x < V) {
      const int xv = x / kV;
      const bool owns = aligned ? (xv < nvec ? (xv >= v0 && xv < v1) : (j == NCH - 1))
                                : (x >= se0 && x < se1);
      if (owns) zx[slot] = load_one<DT>(row, x);
    }
  }
  const int lane = tid & (kWave - 1);
  const int wave = tid / kWave;
  __shared__ double sh_s[kWaves];
  __shared__ float sh_mx[kWaves];
  __shared__ int sh_mi[kWaves];

  // One streaming loop for both kinds of row (the preloaded tile and the two
  // register buffers are shared); the fold is chosen per workgroup.
  const float c = greedy ? 0.0f : temp_scale(T);
  int M = kEmptyM;  // stochastic: (M, s, max)
  double s = 0.0;
  float mx = -INFINITY;
  // greedy: the maximum and its lowest index.  Per vector only its maximum is
  // compared; the vector holding the running maximum is kept whole (bvec, at
  // vector bt + tid) and the index inside it is found once, after the stream.
  // A thread's vectors come in increasing index order, so a strict > keeps the
  // first of equal maxima.
  float bv = -INFINITY;
  int bt = -1;
  u32x4 bvec = u32x4{0u, 0u, 0u, 0u};
  stream_chunk_k1<DT, U, kPre>(rv, v0, v1, tid, pre, [&](const u32x4 *tile, int t0) {
    // only a tile that reaches past v1 is masked (the chunk's last one)
    const bool full = t0 + U * kBlock <= v1;  // uniform per workgroup
    if (!greedy) {
      if (full) {
        fold_tile<DT, U>(tile, c, M, s, mx);
      } else {
        u32x4 m[U];
        mask_tile<DT, U>(tile, t0, v1, tid, m);
        fold_tile<DT, U>(m, c, M, s, mx);
      }
    } else {
      u32x4 m[U];
      if (full) {
#pragma unroll
        for (int u = 0; u < U; ++u) m[u] = tile[u];
      } else {
        mask_tile<DT, U>(tile, t0, v1, tid, m);  // -inf never passes the strict >
      }
#pragma unroll
      for (int u = 0; u < U; ++u) {
        float x[kV];
        widen_vec<DT>(m[u], x);
        float vm = x[0];
#pragma unroll
        for (int e = 1; e < kV; ++e) vm = fmaxf(vm, x[e]);
        const bool take = vm > bv;
        bv = take ? vm : bv;
        bt = take ? t0 + u * kBlock : bt;
        bvec = take ? m[u] : bvec;
      }
    }
  });
  int bi = 0x7fffffff;
  if (greedy) {
    if (bt >= 0) {
      float x[kV];
      widen_vec<DT>(bvec, x);
      int e0 = kV - 1;
#pragma unroll
      for (int e = kV - 1; e >= 0; --e)
        if (x[e] == bv) e0 = e;
      bi = (bt + tid) * kV + e0;
    } else if (v0 + tid < v1) {
      bi = (v0 + tid) * kV;  // every element of this thread's vectors is -inf
    }
  }

  if (!greedy) {
    for (long e = se0 + tid; e < se1; e += kBlock) {
      const float z = load_one<DT>(row, e);
      fold_values<1>(&z, c, M, s, mx);
    }
    // the wave's lanes merged with DPP: the largest M, every lane's sum
    // rescaled to it by an exact power of two, one fp64 sum
    const int Mw = wave_ext_i32<true>(M);
    const double sw = wave_sum(ldexp(s, M - Mw));
    const float mw = wave_max_f32(mx);
    if (lane == 0) {
      sh_s[wave] = sw;
      sh_mx[wave] = mw;
      sh_mi[wave] = Mw;
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
      part[wgid] = pr;
    }
  } else {
    for (long e = se0 + tid; e < se1; e += kBlock) {
      const float z = load_one<DT>(row, e);
      if (z > bv || bi == 0x7fffffff) {
        bv = z;
        bi = static_cast<int>(e);
      }
    }
    // the wave's maximum, then the lowest index holding it (DPP)
    const float vw = wave_max_f32(bv);
    const int iw = wave_ext_i32<false>(bv == vw ? bi : INT_MAX);
    if (lane == 0) {
      sh_mx[wave] = vw;
      sh_mi[wave] = iw;
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
      part[wgid] = pr;
    }
  }
}

// ================================================================== top-k / top-p
// Optional filtering of a stochastic request (the pages name top_p only as a
// serving parameter, so its rule is a reading): every target and draft row of
// the request keeps the tokens with z >= tau, where tau_k is the k-th largest
// logit (equal logits are kept together), tau_p the largest logit value t whose
// tokens {z >= t} hold at least a fraction top_p of the mass that top-k keeps,
// and tau = max(tau_k, tau_p).  The rejection rule then runs on the
// renormalised rows: K2 and K3 treat z < tau as probability zero and use the
// kept mass in place of the row sum.
//
// Four kernels between K1 and K2.  A token's mass is e(z) = 2^(z c - M) with
// the row's integer M from K1; exact sums use the fixed-point integer
// floor(e * 2^fs), fs = 61 - ceil(log2 V), so that they do not depend on the
// order of the additions and a whole row fits 64 bits.
//   FG  k_filter_capture (K1's chunks): appends the order key of every logit
//       within 16 binary orders of magnitude of 2^M (y = z c - M > -16) to the
//       row's candidate list (wave-aggregated slot reservations); a vector
//       whose largest logit is below that is skipped after one test.
//   FD  k_filter_deep_count (K1's chunks of the top-k rows that captured
//       fewer than k logits, whose k-th logit lies below the window): counts of
//       the logits in the bands between the floors y = -18, -20, ..., -40.
//   FC  k_filter_resolve (one workgroup per row): an exact (count, fixed-point
//       mass) histogram of the candidates over 1/32-order bins finds the bin
//       holding the k-th largest logit or the top-p crossing (the candidates
//       are every logit above the window's floor, so the prefixes from the top
//       are exact); that bin's candidates are sorted and scanned group by
//       group.  The top-p target is top_p times the exact top-k mass, or times
//       K1's row sum without top-k.  For a row FD counted, the list is first
//       replaced by a deeper one: the shallowest floor that holds the k-th
//       logit with at most kFCap logits, captured by one pass over the row.
//   FE  k_filter_general (one workgroup per row FC could not resolve: more
//       than kGCap logits captured, a crowded bin, a top-p crossing below the
//       window, or no deeper floor that qualifies):
//   pass 1   exact (count, fixed-point mass) histogram over 2048 bins of y,
//            each 1/32 of a binary order of magnitude, down to y = -64, and
//            one bin below;
//   resolve  the bin where the count reaches k or the mass reaches
//            top_p * kept mass is found by a scan; its logits are gathered in
//            one more pass (a bin holding more than kFCap logits is first split
//            by 2048-way histograms of the order-preserving 32-bit key, one
//            pass each, at most three), sorted, and scanned group by group.
// Both paths apply the same definition; they can differ only where a top-p
// crossing lies within the rounding of the masses (about 1e-7 of the kept
// mass).  The result per row is (tau, kept mass); rows of requests without a
// filter are not touched.
constexpr int kFBlock = 256;  // FC and FE workgroup (FC: three workgroups fit a CU, every row of a batch of 64 x 11 is resident)
constexpr int kFWaves = kFBlock / kWave;
constexpr int kLBlock = 256;  // FG workgroup
constexpr int kFBins = 2048;  // general path: y bins; index kFBins collects y <= -64
constexpr int kFCap = 4096;   // logits sorted and scanned in LDS
constexpr int kLevels = 16;   // the capture window: levels of one binary order of magnitude below 2^M
constexpr int kGCap = 32768;  // logits a row may capture (T = 1.2 rows of a 128K vocabulary fit)
constexpr int kDeep = 12;     // deeper floors y = -18, -20, ..., -40 (FD, FC)
constexpr unsigned kStageVecs = 128;  // 16-byte vectors a wave stages before it offers them (2 KB)

struct alignas(16) FilterStats {
  double s_kept;  // sum of 2^(z c - M) over the kept tokens
  float tau;      // tokens with z >= tau are kept
  int pad;
};

// Device buffers of the filter kernels (inside the workspace).
struct FilterWork {
  unsigned *ncand;   // [slots] logits captured (cleared by K1)
  unsigned *cand;    // [slots][kGCap] their order keys
  unsigned *dcount;  // [slots][NS][kDeep + 1] FD's per-chunk counts above the floors
};

// Whether a request with top_k kr and top_p pr filters, with its k (0: none)
// and p (1: none).  Values outside the documented ranges switch the
// corresponding filter off.
__device__ __forceinline__ bool filter_params(int kr, float pr, int V, int &k, float &p) {
  k = (kr > 0 && kr < V) ? kr : 0;
  p = (pr > 0.0f && pr < 1.0f) ? pr : 1.0f;
  return k > 0 || p < 1.0f;
}

// ================================================================== K2
constexpr int kK2Batch = 8;  // chunk partials fetched together per row

struct DecideShared {
  double s[2 * SV_GAMMA_MAX + 1];
  float tau[2 * SV_GAMMA_MAX + 1];
  int M[2 * SV_GAMMA_MAX + 1];
  int arg[2 * SV_GAMMA_MAX + 1];
  int k;
  SelParams sp;
};

// The decision for request b, computed by one 256-thread workgroup: merge the
// chunk partials of each row in chunk order, evaluate the acceptance of each
// draft, find the first rejection.  Every workgroup of a request computes the
// same result (the arithmetic is deterministic); only the `writer` workgroup
// stores the outputs and the sampling parameters.  Returns them in sh.sp.
template <int DT, bool FILT>
__device__ __forceinline__ void decide_request(
    const void *__restrict__ target, const void *__restrict__ draft,
    const int32_t *__restrict__ tokens, const float *__restrict__ u_accept,
    const float *__restrict__ temps, float scalar_T, const int32_t *__restrict__ lens, int gamma,
    int V, int NS, const Partial *__restrict__ part, const float *__restrict__ zx,
    const int32_t *__restrict__ topk, const float *__restrict__ topp, const FilterStats *__restrict__ fst,
    int32_t *__restrict__ accepted_count, int32_t *__restrict__ out_tokens,
    SelParams *__restrict__ sel, const sv_debug &dbg_in, int b, bool writer, DecideShared &sh,
    bool drawn_elsewhere = false) {
  const int tid = threadIdx.x;
  const int rows = 2 * gamma + 1;
  const int g = request_len(lens, gamma, b);
  const float T = request_T(temps, scalar_T, b);
  // the filter parameters are fetched together with T (one round trip)
  const int fkr = FILT && topk ? topk[b] : 0;
  const float fpr = FILT && topp ? topp[b] : 1.0f;
  const bool greedy = !(T > 0.0f);
  const float c = greedy ? 0.0f : temp_scale(T);
  int fk;
  float fp;
  const bool filtered = FILT && filter_params(fkr, fpr, V, fk, fp) && !greedy;
  sv_debug dbg = dbg_in;
  if (!writer) memset(&dbg, 0, sizeof dbg);
  double *sh_s = sh.s;
  int *sh_M = sh.M;
  int *sh_arg = sh.arg;
  int &sh_k = sh.k;

  // thread i < g also evaluates draft i: its id, its uniform, and the two logits
  // at it (picked up by K1), fetched together with the row partials below
  int x = -1;
  float zpx = 0.0f, zqx = 0.0f, ua = 0.0f;
  if (tid < g) {
    x = tokens[static_cast<long>(b) * gamma + tid];
    if (!greedy) {
      zpx = zx[static_cast<long>(b) * rows + tid];
      zqx = zx[static_cast<long>(b) * rows + gamma + 1 + tid];
      ua = u_accept[static_cast<long>(b) * gamma + tid];
    }
  }

  // merge the tile partials of each needed row, tiles in increasing order
  if (tid < rows) {
    const int r = tid;
    const bool is_target = r <= gamma;
    const int i = is_target ? r : r - gamma - 1;
    const bool needed = is_target ? (i <= g) : (!greedy && i < g);
    if (needed) {
      const Partial *pp = part + (static_cast<long>(b) * rows + r) * NS;
      // the row's filter statistics (written for every filtered row), fetched
      // together with the partials
      FilterStats fsr;
      if (FILT && filtered) fsr = fst[static_cast<long>(b) * rows + r];
      int M = kEmptyM;
      double s = 0.0;
      float mx = -INFINITY;
      float v = -INFINITY;
      int ix = 0x7fffffff;
      for (int j0 = 0; j0 < NS; j0 += kK2Batch) {
        Partial buf[kK2Batch];
#pragma unroll
        for (int u = 0; u < kK2Batch; ++u)
          if (j0 + u < NS) buf[u] = pp[j0 + u];
#pragma unroll
        for (int u = 0; u < kK2Batch; ++u) {
          if (j0 + u < NS) {
            if (!greedy) merge_sm(M, s, mx, buf[u].mi, buf[u].s, buf[u].mx);
            else merge_arg(v, ix, buf[u].mx, buf[u].mi);
          }
        }
      }
      if (!greedy) {
        float tau = -INFINITY;
        if (FILT && filtered) {  // the kept mass replaces the row sum
          s = fsr.s_kept;
          tau = fsr.tau;
        }
        sh_M[r] = M;
        sh_s[r] = s;
        sh.tau[r] = tau;
        if (dbg.row_max) dbg.row_max[static_cast<long>(b) * rows + r] = mx;
        if (dbg.row_sum)  // sum_v exp((z_v - max)/T) = s * 2^(M - max c)
          dbg.row_sum[static_cast<long>(b) * rows + r] =
              s * exp2(static_cast<double>(M) - static_cast<double>(mx) * static_cast<double>(c));
      } else {
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
      if (x < 0 || x >= V) {
        reject = true;  // a draft id outside the vocabulary is rejected, never dereferenced
      } else if (greedy) {
        reject = (x != sh_arg[tid]);
      } else {
        const double cd = static_cast<double>(c);
        // p_i(x) / q_i(x) = 2^((zp - zq) c - (Mp - Mq)) * s'_q / s'_p, in fp64; the
        // logit difference is exact and the exponent stays O(1)
        const int Mp = sh_M[tid], Mq = sh_M[gamma + 1 + tid];
        const double sp_ = sh_s[tid], sq_ = sh_s[gamma + 1 + tid];
        // a token cut by the filter has probability zero; q(x) = 0 accepts
        // when p(x) > 0 and rejects otherwise
        const bool pin = !FILT || zpx >= sh.tau[tid], qin = !FILT || zqx >= sh.tau[gamma + 1 + tid];
        double a;
        if (!qin) {
          a = pin ? 1.0 : 0.0;
        } else if (!pin) {
          a = 0.0;
        } else {
          const double d = (static_cast<double>(zpx) - static_cast<double>(zqx)) * cd -
                           static_cast<double>(Mp - Mq);
          const double ratio = exp2(d) * (sq_ / sp_);
          a = ratio < 1.0 ? ratio : 1.0;
        }
        reject = !(static_cast<double>(ua) < a);
        const long o = static_cast<long>(b) * gamma + tid;
        if (dbg.p_draft) dbg.p_draft[o] = pin ? exp2(static_cast<double>(zpx) * cd - Mp) / sp_ : 0.0;
        if (dbg.q_draft) dbg.q_draft[o] = qin ? exp2(static_cast<double>(zqx) * cd - Mq) / sq_ : 0.0;
        if (dbg.accept_prob) dbg.accept_prob[o] = a;
      }
    }
    const unsigned long long rej = __ballot(reject);
    if (tid == 0) sh_k = rej ? (__ffsll(static_cast<long long>(rej)) - 1) : g;
  }
  __syncthreads();
  const int k = sh_k;

  // accepted prefix, the greedy replacement / bonus, -1 padding; a stochastic
  // request's token at k is left to the draw when another workgroup of the
  // same kernel makes it (drawn_elsewhere), which this store must not overwrite
  if (writer) {
    for (int t = tid; t <= gamma; t += kBlock) {
      int32_t v = -1;
      if (t < k) v = tokens[static_cast<long>(b) * gamma + t];
      else if (t == k && greedy) v = sh_arg[k];
      else if (t == k && drawn_elsewhere) continue;
      out_tokens[static_cast<long>(b) * (gamma + 1) + t] = v;
    }
  }
  if (tid == 0) {
    if (writer) accepted_count[b] = k;
    SelParams sp;
    sp.k = k;
    sp.c = c;
    sp.tau_p = sp.tau_q = -INFINITY;
    if (greedy) {
      sp.mode = 0;
      sp.negMp = sp.negMq = 0.0f;
      sp.r = 0.0f;
      sp.ip = 0.0;
    } else {
      sp.mode = (k < g) ? 1 : 2;
      sp.negMp = -static_cast<float>(sh_M[k]);
      sp.ip = 1.0 / sh_s[k];
      sp.tau_p = sh.tau[k];
      if (k < g) {
        sp.negMq = -static_cast<float>(sh_M[gamma + 1 + k]);
        sp.r = static_cast<float>(sh_s[k] / sh_s[gamma + 1 + k]);
        sp.tau_q = sh.tau[gamma + 1 + k];
      } else {
        sp.negMq = 0.0f;
        sp.r = 0.0f;
      }
    }
    if (writer) sel[b] = sp;
    sh.sp = sp;
  }
  __syncthreads();
}

// ================================================================== K3
// Sampling at position k of a stochastic request.  With e_p = 2^(z_p c - M_p),
// e_q = 2^(z_q c - M_q) and r = s'_p / s'_q,
//   p(v) - q(v) = (e_p(v) - r e_q(v)) / s'_p,
// so the residual is handled in units of the target row's scale s'_p: a common
// scale does not move the normalised CDF, and sampling never divides by s'_p.
// The bonus (k == gamma_b) samples w = e_p.  The sum of e_p is kept alongside
// for the zero-residual-mass fallback to p_k.
//
// The row is cut into sub-chunks of kSub = 2048 tokens, one wave each, 32
// tokens per lane.  K3a writes the mass of every sub-chunk; K3b (one wave per
// request) finds the sub-chunk whose prefix crosses u*Z and then the token in it.
constexpr int kLaneElems = kSub / kWave;  // 32

// FILT: the request may be filtered (top-k / top-p); tokens below the cut carry
// no mass.  Unfiltered launches compile without the compares.
// USEQ: the residual at a rejection (sp.mode == 1); otherwise the bonus row.
template <bool FILT, bool USEQ>
__device__ __forceinline__ void residual_value_of(const SelParams &sp, float zp, float zq, float &w, float &p) {
  float ep = __builtin_amdgcn_exp2f(fmaf(zp, sp.c, sp.negMp));  // -inf -> 0
  if (FILT && !(zp >= sp.tau_p)) ep = 0.0f;
  p = ep;
  if constexpr (USEQ) {
    float eq = __builtin_amdgcn_exp2f(fmaf(zq, sp.c, sp.negMq));
    if (FILT && !(zq >= sp.tau_q)) eq = 0.0f;
    w = fmaxf(0.0f, fmaf(-eq, sp.r, ep));
  } else {
    w = ep;
  }
}

template <bool FILT>
__device__ __forceinline__ void residual_value(const SelParams &sp, float zp, float zq, float &w,
                                               float &p) {
  if (sp.mode == 1) residual_value_of<FILT, true>(sp, zp, zq, w, p);
  else residual_value_of<FILT, false>(sp, zp, zq, w, p);
}

// The 32 logits of one lane in a sub-chunk starting at token `base`.
// INTERLEAVED: vector u of the lane is vector u*64 + lane of the sub-chunk
//   (each load instruction of the wave reads one contiguous 1 KiB run);
// otherwise the lane's 32 tokens are contiguous (base + lane*32 + k), which the
//   in-sub-chunk scan needs.  Tokens at or beyond V read as -inf.
template <int DT, bool INTERLEAVED>
__device__ __forceinline__ void load_lane32(const void *row, bool aligned, long base, int lane, long V,
                                            float *z, int *idx) {
  constexpr int kV = Elem<DT>::kVec;
#pragma unroll
  for (int u = 0; u < kLaneElems / kV; ++u) {
    const long e0 = INTERLEAVED ? base + static_cast<long>(u * kWave + lane) * kV
                                : base + static_cast<long>(lane) * kLaneElems + u * kV;
    load_vec_guarded<DT>(row, aligned, e0, V, z + u * kV);
    if (idx) {
#pragma unroll
      for (int e = 0; e < kV; ++e) idx[u * kV + e] = static_cast<int>(e0 + e);
    }
  }
}

struct RowPair {
  const void *trow, *drow;
  bool aligned;
};

template <int DT>
__device__ __forceinline__ RowPair selected_rows(const void *target, const void *draft, int gamma, int V,
                                                 int b, const SelParams &sp) {
  RowPair rp;
  rp.trow = static_cast<const char *>(target) +
            (static_cast<long>(b) * (gamma + 1) + sp.k) * V * Elem<DT>::kBytes;
  rp.drow = (sp.mode == 1) ? static_cast<const void *>(static_cast<const char *>(draft) +
                                                       (static_cast<long>(b) * gamma + sp.k) * V *
                                                           Elem<DT>::kBytes)
                           : nullptr;
  rp.aligned = ((reinterpret_cast<uintptr_t>(rp.trow) | reinterpret_cast<uintptr_t>(rp.drow)) & 15u) == 0;
  return rp;
}

// Raw 16-byte vectors holding one lane's 32 tokens of a sub-chunk, interleaved
// layout (vector u of the lane is vector u*64 + lane of the sub-chunk, so each
// load instruction of the wave reads one contiguous 1 KiB run).  Tokens at or
// beyond V, and every token of a row that is not 16-byte aligned, are read one
// by one; out-of-range tokens hold -inf.
template <int DT>
__device__ __forceinline__ u32x4 pack_guarded(const char *row, long e0, long V) {
  uint32_t w[4];
  if constexpr (DT == SV_F32) {
#pragma unroll
    for (int e = 0; e < 4; ++e)
      w[e] = (e0 + e < V) ? reinterpret_cast<const uint32_t *>(row)[e0 + e] : 0xff800000u;
  } else {
    const uint16_t *h = reinterpret_cast<const uint16_t *>(row);
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const uint32_t lo = (e0 + 2 * e < V) ? h[e0 + 2 * e] : 0xff80u;
      const uint32_t hi = (e0 + 2 * e + 1 < V) ? h[e0 + 2 * e + 1] : 0xff80u;
      w[e] = lo | (hi << 16);
    }
  }
  return u32x4{w[0], w[1], w[2], w[3]};
}

template <int DT>
__device__ __forceinline__ void load_lane_raw(const void *row, bool aligned, long base, int lane, long V,
                                              u32x4 *raw) {
  constexpr int kV = Elem<DT>::kVec;
  const char *r = static_cast<const char *>(row);
#pragma unroll
  for (int u = 0; u < kLaneElems / kV; ++u) {
    const long e0 = base + static_cast<long>(u * kWave + lane) * kV;
    raw[u] = (aligned && e0 + kV <= V)
                 ? *reinterpret_cast<const u32x4 *>(r + e0 * Elem<DT>::kBytes)
                 : pack_guarded<DT>(r, e0, V);
  }
}

// One lane's 32 tokens of a sub-chunk that lies wholly inside a 16-byte aligned
// row, in the interleaved layout of load_lane_raw, with no guards.
template <int DT>
__device__ __forceinline__ void load_lane_fast(const void *row, long base, int lane, u32x4 *raw) {
  constexpr int kV = Elem<DT>::kVec;
  const u32x4 *r = reinterpret_cast<const u32x4 *>(static_cast<const char *>(row) + base * Elem<DT>::kBytes);
#pragma unroll
  for (int u = 0; u < kLaneElems / kV; ++u) raw[u] = r[u * kWave + lane];
}

// A sub-chunk mass as a hand-over word: the fp64 bits plus one, so that a
// mass (never negative) is never the cleared value 0.
__device__ __forceinline__ unsigned long long sub_mass_word(double m) {
  return static_cast<unsigned long long>(__double_as_longlong(m)) + 1ull;
}

// The masses of the wave's SPW consecutive sub-chunks [first, ...) of the row
// pair to sample (USEQ: residual at a rejection, else the bonus row), loading
// sub-chunk t+1 while sub-chunk t is reduced.  FAST: every one of them lies
// wholly inside an aligned row.
template <int DT, bool FILT, bool FAST, bool USEQ, bool COH>
__device__ __forceinline__ void mass_pass(const RowPair &rp, const SelParams &sp, int first, int SPW, int NSUB,
                                          int V, int lane, SubSums *__restrict__ out, double *lds_w = nullptr,
                                          double *lds_p = nullptr) {
  constexpr int kN = kLaneElems / Elem<DT>::kVec;
  auto load = [&](const void *row, int sub, u32x4 *dst) {
    if constexpr (FAST) load_lane_fast<DT>(row, static_cast<long>(sub) * kSub, lane, dst);
    else load_lane_raw<DT>(row, rp.aligned, static_cast<long>(sub) * kSub, lane, V, dst);
  };
  u32x4 tc[kN], dc[kN], tn[kN], dn[kN];
  load(rp.trow, first, tc);
  if constexpr (USEQ) load(rp.drow, first, dc);
  for (int t = 0; t < SPW; ++t) {
    const int sub = first + t;
    if (sub >= NSUB) break;
    if (t + 1 < SPW && sub + 1 < NSUB) {
      load(rp.trow, sub + 1, tn);
      if constexpr (USEQ) load(rp.drow, sub + 1, dn);
    }
    float aw[8], ap[8];
#pragma unroll
    for (int e = Elem<DT>::kVec; e < 8; ++e) aw[e] = ap[e] = 0.0f;  // unused by 4-wide vectors
#pragma unroll
    for (int u = 0; u < kN; ++u) {
      float zp[Elem<DT>::kVec], zq[Elem<DT>::kVec];
      widen_vec<DT>(tc[u], zp);
      if constexpr (USEQ) widen_vec<DT>(dc[u], zq);
#pragma unroll
      for (int e = 0; e < Elem<DT>::kVec; ++e) {
        float w, p;
        residual_value_of<FILT, USEQ>(sp, zp[e], USEQ ? zq[e] : 0.0f, w, p);
        if (u == 0) {  // the first vector's terms start the sums (no add of zero)
          aw[e & 7] = w;
          ap[e & 7] = p;
        } else {
          aw[e & 7] += w;
          ap[e & 7] += p;
        }
      }
    }
    const float lw = ((aw[0] + aw[1]) + (aw[2] + aw[3])) + ((aw[4] + aw[5]) + (aw[6] + aw[7]));
    const float lp = ((ap[0] + ap[1]) + (ap[2] + ap[3])) + ((ap[4] + ap[5]) + (ap[6] + ap[7]));
    const double sw = wave_sum(static_cast<double>(lw));
    const double spp = wave_sum(static_cast<double>(lp));
    if (lane == 0) {
      if (lds_w) {  // the only workgroup of its request: the masses stay in LDS
        lds_w[sub] = sw;
        lds_p[sub] = spp;
      } else if constexpr (COH) {  // hand-over words read by other workgroups
        unsigned long long *w = reinterpret_cast<unsigned long long *>(out + sub);
        put<true>(w, sub_mass_word(sw));
        put<true>(w + 1, sub_mass_word(spp));
      } else {
        SubSums ss;
        ss.w = sw;
        ss.p = spp;
        out[sub] = ss;
      }
    }
#pragma unroll
    for (int u = 0; u < kN; ++u) {
      tc[u] = tn[u];
      if constexpr (USEQ) dc[u] = dn[u];
    }
  }
}

// The draw inside one 2048-token sub-chunk from the vectors a wave holds in
// the interleaved layout of load_lane_fast (vector u of a lane is vector
// u*64 + lane of the sub-chunk, so the sub-chunk's order is vector slot, then
// lane, then element): per-vector sums, a wave scan per slot, the slot whose
// prefix crosses the target, the lane by a ballot, the element by the lane.
// Rounding past the sub-chunk's end: its last token with mass.  sub_tok: the
// sub-chunk's first token; base_mass: the mass before it.  Called by the whole
// wave; one lane writes the token.
template <int DT, bool FILT>
__device__ __forceinline__ void draw_held(const u32x4 *tv, const u32x4 *dv, const SelParams &sp, bool use_p,
                                          long sub_tok, double base_mass, double target_mass, int lane,
                                          int32_t *dst) {
  constexpr int kV = Elem<DT>::kVec;
  constexpr int kN = kLaneElems / kV;
  auto vals_of = [&](u32x4 t, u32x4 d, float *v) {
    float zp[kV], zq[kV];
    widen_vec<DT>(t, zp);
    if (sp.mode == 1) widen_vec<DT>(d, zq);
#pragma unroll
    for (int e = 0; e < kV; ++e) {
      float w, p;
      residual_value<FILT>(sp, zp[e], sp.mode == 1 ? zq[e] : 0.0f, w, p);
      v[e] = use_p ? p : w;
    }
  };
  float vs[kN];
  double incl[kN];
  int us = -1, ulast = -1;
  double run = base_mass, at = base_mass, at_last = base_mass;
#pragma unroll
  for (int u = 0; u < kN; ++u) {
    float v[kV];
    vals_of(tv[u], sp.mode == 1 ? dv[u] : tv[u], v);
    float t;
    if constexpr (kV == 8) t = ((v[0] + v[1]) + (v[2] + v[3])) + ((v[4] + v[5]) + (v[6] + v[7]));
    else t = (v[0] + v[1]) + (v[2] + v[3]);
    vs[u] = t;
    incl[u] = wave_scan(static_cast<double>(t), lane);
    const double tot = lane_value(incl[u], kWave - 1);
    if (tot > 0.0) {
      if (us < 0 && run + tot > target_mass) {
        us = u;
        at = run;
      }
      ulast = u;
      at_last = run;
    }
    run += tot;
  }
  if (us < 0) {
    us = ulast >= 0 ? ulast : 0;
    at = ulast >= 0 ? at_last : base_mass;
  }
  // the slot's values, selected without indexing the register arrays by a
  // runtime value (that would move them to scratch memory)
  float vu = 0.0f;
  double iu = 0.0;
  u32x4 tu = tv[0], du = tv[0];
#pragma unroll
  for (int u = 0; u < kN; ++u)
    if (u == us) {
      vu = vs[u];
      iu = incl[u];
      tu = tv[u];
      if (sp.mode == 1) du = dv[u];
    }
  const double excl = at + (iu - static_cast<double>(vu));
  const unsigned long long hit = __ballot(vu > 0.0f && excl + static_cast<double>(vu) > target_mass);
  const unsigned long long has = __ballot(vu > 0.0f);
  const int L = hit ? __ffsll(static_cast<long long>(hit)) - 1 : (has ? 63 - __clzll(static_cast<long long>(has)) : 0);
  if (lane == L) {
    float v[kV];
    vals_of(tu, du, v);
    double acc = excl;
    int tok = -1, lastm = -1;
#pragma unroll
    for (int e = 0; e < kV; ++e) {
      if (v[e] > 0.0f) {
        lastm = e;
        acc += static_cast<double>(v[e]);
        if (tok < 0 && target_mass < acc) tok = e;
      }
    }
    if (tok < 0) tok = lastm >= 0 ? lastm : 0;
    *dst = static_cast<int32_t>(sub_tok + static_cast<long>(us * kWave + L) * kV + tok);
  }
}

// The draw of request b at position sp.k from its sub-chunk masses, read
// through mass(s, p) (p: the bonus row's mass of p, else the residual mass w);
// with subs_per_wg > 0 only workgroup wg's sub-chunks are drawn from here;
// w0, p0 are the masses of sub-chunks [0, 64) of this lane, fetched early by
// the caller.  Every wave redundantly finds the total mass Z (zero residual
// mass falls back to p_k) and the lowest sub-chunk with mass whose inclusive
// prefix exceeds u*Z; then wave w scans tokens [512 w, 512 w + 512) of that
// sub-chunk, 8 contiguous tokens per lane, and the lowest token with mass whose
// running prefix exceeds u*Z is emitted.  One 256-thread workgroup, every
// thread present.
template <int DT, bool FILT, typename Mass>
__device__ __forceinline__ void select_token(const void *__restrict__ target, const void *__restrict__ draft,
                                             float u, int gamma, int V, int NSUB, int b, const SelParams &sp,
                                             double w0, double p0, Mass &&mass, int32_t *__restrict__ out_tokens,
                                             double *__restrict__ dbg_mass, int wg = 0, int subs_per_wg = 0) {
  const int tid = threadIdx.x, lane = tid & (kWave - 1), wave = tid / kWave;
  double Zw = wave_sum(w0), Zp = wave_sum(p0);
  for (int base = kWave; base < NSUB; base += kWave) {
    const int s = base + lane;
    Zw += wave_sum(s < NSUB ? mass(s, false) : 0.0);
    Zp += wave_sum(s < NSUB ? mass(s, true) : 0.0);
  }
  const bool use_p = !(Zw > 0.0);  // zero residual mass: fall back to p_k
  const double Z = use_p ? Zp : Zw;
  const double target_mass = static_cast<double>(u) * Z;

  int sub = -1;
  double base_mass = 0.0, run = 0.0;
  for (int base = 0; base < NSUB; base += kWave) {
    const int s = base + lane;
    const double v = (base == 0) ? (use_p ? p0 : w0) : (s < NSUB ? mass(s, use_p) : 0.0);
    const double incl = wave_scan(v, lane);
    const unsigned long long hit = __ballot(s < NSUB && v > 0.0 && run + incl > target_mass);
    if (hit) {
      const int L = __ffsll(static_cast<long long>(hit)) - 1;
      sub = base + L;
      base_mass = run + lane_value(incl - v, L);
      break;
    }
    run += lane_value(incl, kWave - 1);
  }
  if (sub < 0) {  // rounding left u*Z at the very end: the last sub-chunk with mass
    run = 0.0;
    for (int base = 0; base < NSUB; base += kWave) {
      const int s = base + lane;
      const double v = s < NSUB ? mass(s, use_p) : 0.0;
      const double incl = wave_scan(v, lane);
      const unsigned long long has = __ballot(s < NSUB && v > 0.0);
      if (has) {
        const int L = 63 - __clzll(static_cast<long long>(has));
        sub = base + L;
        base_mass = run + lane_value(incl - v, L);
      }
      run += lane_value(incl, kWave - 1);
    }
    if (sub < 0) {
      sub = 0;
      base_mass = 0.0;
    }
  }

  // with subs_per_wg, only the workgroup that computed the sub-chunk's mass
  // goes on (its data is in this XCD's L2); the same result in every wave
  if (subs_per_wg > 0 && sub / subs_per_wg != wg) return;

  // tokens [first, first + 8) of this lane, in order through waves and lanes
  const RowPair rp = selected_rows<DT>(target, draft, gamma, V, b, sp);
  const long first = static_cast<long>(sub) * kSub + wave * (kSub / kWaves) + lane * 8;
  float zp[8], zq[8];
  load_vec_guarded<DT>(rp.trow, rp.aligned, first, V, zp);
  if constexpr (DT == SV_F32) load_vec_guarded<DT>(rp.trow, rp.aligned, first + 4, V, zp + 4);
  if (sp.mode == 1) {
    load_vec_guarded<DT>(rp.drow, rp.aligned, first, V, zq);
    if constexpr (DT == SV_F32) load_vec_guarded<DT>(rp.drow, rp.aligned, first + 4, V, zq + 4);
  }
  float vals[8];
  double lsum = 0.0;
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    float w, p;
    residual_value<FILT>(sp, zp[e], sp.mode == 1 ? zq[e] : 0.0f, w, p);
    vals[e] = use_p ? p : w;
    lsum += static_cast<double>(vals[e]);
  }
  const double incl = wave_scan(lsum, lane);
  __shared__ double sh_tot[kWaves];
  __shared__ int sh_pick[kWaves];
  __shared__ int sh_last[kWaves];
  if (lane == kWave - 1) sh_tot[wave] = incl;
  __syncthreads();
  double before = base_mass;
  for (int w = 0; w < wave; ++w) before += sh_tot[w];
  double acc = before + (incl - lsum);
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
  const unsigned long long has = __ballot(last_pos >= 0);
  const int Lp = props ? __ffsll(static_cast<long long>(props)) - 1 : -1;
  const int Lh = has ? 63 - __clzll(static_cast<long long>(has)) : -1;
  // the winning token of this wave (first proposal), and its last token with mass
  const int pick = Lp >= 0 ? static_cast<int>(__shfl(first + cand, Lp)) : -1;
  const int lastm = Lh >= 0 ? static_cast<int>(__shfl(first + last_pos, Lh)) : -1;
  if (lane == 0) {
    sh_pick[wave] = pick;
    sh_last[wave] = lastm;
  }
  __syncthreads();
  if (tid == 0) {
    int tok = -1;
    for (int w = 0; w < kWaves && tok < 0; ++w) tok = sh_pick[w];
    // rounding left u*Z past the sub-chunk: its last token with mass
    for (int w = kWaves - 1; w >= 0 && tok < 0; --w) tok = sh_last[w];
    if (tok < 0) tok = static_cast<int>(static_cast<long>(sub) * kSub);
    out_tokens[static_cast<long>(b) * (gamma + 1) + sp.k] = tok;
    if (dbg_mass) dbg_mass[b] = Z * sp.ip;
  }
}


// Requests whose sub-chunk masses fit workgroup 0's LDS when K2 also draws.
constexpr int kSelMaxSub = 512;  // V <= 2^20

// K2 (decide) fused with K3a (mass): NW workgroups per request.  Each one
// recomputes the request's decision (cheap and deterministic) and workgroup 0
// stores it; then every wave writes the masses of SPW consecutive 2048-token
// sub-chunks of the row pair to sample, loading sub-chunk t+1 while it reduces
// sub-chunk t.
//
// SEL: the draw as well (K3b is not launched).  The masses go out as
// hand-over words (cleared by K1 in the same call) and are polled by the first
// wave of a workgroup until all have arrived (bounded: past the limit the
// token is -1).  With `owner` (a grid that is resident at once) every
// workgroup of the request polls, finds the sub-chunk holding u*Z, and the one
// that computed its mass draws the token in it as K3b does, from its own XCD's
// L2; otherwise workgroup 0 alone polls and draws, so that waiting workgroups
// do not hold back the dispatch of later ones.  The earliest request not yet
// done never waits for a workgroup dispatched after a later request's, so the
// waits end.
// bf16 rows: at most 128 registers (4 waves per SIMD, 4 workgroups per CU),
// the residency the drawing mode is chosen for
template <int DT, bool FILT, bool SEL>
__global__ __launch_bounds__(kBlock, DT == SV_BF16 ? 4 : 1) void k2_decide_mass(
    const void *__restrict__ target, const void *__restrict__ draft,
    const int32_t *__restrict__ tokens, const float *__restrict__ u_accept,
    const float *__restrict__ temps, float scalar_T, const int32_t *__restrict__ lens, int gamma,
    int V, int NS, int NSUB, int NW, int SPW, const Partial *__restrict__ part,
    const float *__restrict__ zx, const int32_t *__restrict__ topk, const float *__restrict__ topp,
    const FilterStats *__restrict__ fst, int32_t *__restrict__ accepted_count,
    int32_t *__restrict__ out_tokens, SelParams *__restrict__ sel, SubSums *__restrict__ sums,
    const float *__restrict__ u_sample, bool owner, sv_debug dbg) {
  const int b = blockIdx.x / NW;
  const int wg = blockIdx.x - b * NW;
  // greedy requests need the decision only (workgroup 0)
  if (wg > 0 && !(request_T(temps, scalar_T, b) > 0.0f)) return;
  __shared__ DecideShared sh;
  decide_request<DT, FILT>(target, draft, tokens, u_accept, temps, scalar_T, lens, gamma, V, NS, part, zx,
                           topk, topp, fst, accepted_count, out_tokens, sel, dbg, b, wg == 0, sh, SEL);
  const SelParams sp = sh.sp;
  const int first = (wg * kWaves + static_cast<int>(threadIdx.x) / kWave) * SPW;
  const int lane = threadIdx.x & (kWave - 1);
  SubSums *out = sums + static_cast<long>(b) * NSUB;
  __shared__ double sh_w[SEL ? kSelMaxSub : 1], sh_p[SEL ? kSelMaxSub : 1];
  // a request with one workgroup keeps its masses in LDS (no hand-over)
  double *lw = SEL && NW == 1 ? sh_w : nullptr, *lp = SEL && NW == 1 ? sh_p : nullptr;
  if (sp.mode != 0 && first < NSUB) {  // uniform per wave; no barrier inside
    const RowPair rp = selected_rows<DT>(target, draft, gamma, V, b, sp);
    // the wave's sub-chunks lie wholly inside an aligned row: straight-line
    // loads, so that the arithmetic on each vector can start as it arrives
    const bool fast = rp.aligned && static_cast<long>(min(first + SPW, NSUB)) * kSub <= static_cast<long>(V);
    if (sp.mode == 1) {
      if (fast) mass_pass<DT, FILT, true, true, SEL>(rp, sp, first, SPW, NSUB, V, lane, out, lw, lp);
      else mass_pass<DT, FILT, false, true, SEL>(rp, sp, first, SPW, NSUB, V, lane, out, lw, lp);
    } else {
      if (fast) mass_pass<DT, FILT, true, false, SEL>(rp, sp, first, SPW, NSUB, V, lane, out, lw, lp);
      else mass_pass<DT, FILT, false, false, SEL>(rp, sp, first, SPW, NSUB, V, lane, out, lw, lp);
    }
  }
  if constexpr (SEL) {
    if (sp.mode == 0 || (!owner && wg != 0)) return;  // uniform per workgroup
    __shared__ int s_late;
    const unsigned long long *words = reinterpret_cast<const unsigned long long *>(out);
    if (NW == 1) {
      if (threadIdx.x == 0) s_late = 0;
    } else if (threadIdx.x < kWave) {
      bool late = false;
      for (int j0 = 0; j0 < 2 * NSUB; j0 += kWave) {
        const int j = j0 + lane;
        unsigned long long word = 0;
        for (unsigned it = 0;; ++it) {
          if (j < 2 * NSUB) word = get<true>(words + j);
          if (__all(j >= 2 * NSUB || word != 0ull)) break;
          if (it >= kSpinLimit) {
            late = true;
            break;
          }
          __builtin_amdgcn_s_sleep(1);
        }
        if (j < 2 * NSUB) {
          const double m = __longlong_as_double(static_cast<long long>(word - 1ull));
          if (j & 1) sh_p[j >> 1] = m;
          else sh_w[j >> 1] = m;
        }
      }
      if (lane == 0) s_late = late;
    }
    __syncthreads();
    if (s_late) {  // a mass never arrived: no token (uniform per workgroup)
      if (threadIdx.x == 0 && wg == 0) out_tokens[static_cast<long>(b) * (gamma + 1) + sp.k] = -1;
      return;
    }
    const double w0 = lane < NSUB ? sh_w[lane] : 0.0, p0 = lane < NSUB ? sh_p[lane] : 0.0;
    select_token<DT, FILT>(target, draft, u_sample[b], gamma, V, NSUB, b, sp, w0, p0,
                           [&](int s, bool p) { return p ? sh_p[s] : sh_w[s]; }, out_tokens, dbg.residual_mass,
                           wg, owner ? kWaves * SPW : 0);
  }
}

// K3b: one workgroup per request, the draw from the masses K2 wrote.
template <int DT, bool FILT>
__global__ __launch_bounds__(kBlock) void k3_select(
    const void *__restrict__ target, const void *__restrict__ draft,
    const float *__restrict__ u_sample, int gamma, int V, int NSUB,
    const SelParams *__restrict__ sel, const SubSums *__restrict__ sums,
    int32_t *__restrict__ out_tokens, double *__restrict__ dbg_mass) {
  const int b = blockIdx.x;
  const int lane = threadIdx.x & (kWave - 1);
  const SubSums *bs = sums + static_cast<long>(b) * NSUB;
  // the first 64 sub-chunk masses are fetched together with the parameters
  const double w0 = (lane < NSUB) ? bs[lane].w : 0.0;
  const double p0 = (lane < NSUB) ? bs[lane].p : 0.0;
  const SelParams sp = sel[b];
  if (sp.mode == 0) return;  // uniform per workgroup
  select_token<DT, FILT>(target, draft, u_sample[b], gamma, V, NSUB, b, sp, w0, p0,
                         [&](int s, bool p) { return p ? bs[s].p : bs[s].w; }, out_tokens, dbg_mass);
}

// ================================================================== top-k / top-p kernel
// Order-preserving key of a logit (larger value, larger key); -0 is folded
// into +0 so that equal values have equal keys.
__device__ __forceinline__ uint32_t order_key(float z) {
  const uint32_t u = __float_as_uint(z == 0.0f ? 0.0f : z);
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

__device__ __forceinline__ float key_value(uint32_t k) {
  return __uint_as_float((k & 0x80000000u) ? (k & 0x7fffffffu) : ~k);
}

// y bin of a logit: 0 holds the top 1/32 of an order of magnitude below 2^M.
__device__ __forceinline__ int ybin(float z, float c, float negM) {
  const float y = fmaf(z, c, negM);
  if (!(y > -64.0f)) return kFBins;
  const float t = floorf(-32.0f * y);
  return t <= 0.0f ? 0 : static_cast<int>(fminf(t, static_cast<float>(kFBins - 1)));
}

// floor(2^(z c - M) * 2^fs), the exponential being the same v_exp_f32 as K1's.
__device__ __forceinline__ unsigned long long fixed_mass(float z, float c, float negM, int fs) {
  const uint32_t bits = __float_as_uint(__builtin_amdgcn_exp2f(fmaf(z, c, negM)));
  const int ex = static_cast<int>(bits >> 23);  // biased exponent of a value >= 0
  if (ex == 0) return 0ull;                     // zero or below 2^-126
  const unsigned long long mant = (bits & 0x7fffffu) | 0x800000u;
  const int sh = ex - 150 + fs;                 // value = mant * 2^(ex - 150)
  if (sh >= 0) return mant << sh;
  return sh > -24 ? (mant >> -sh) : 0ull;
}

// LDS shared by the scans of both filter kernels.
struct FilterScratch {
  unsigned long long red[2 * kFWaves];
  unsigned long long pick_c, pick_m, res_m;
  unsigned klo, khi, nkeys;
  int pick;
};

struct GeneralShared {
  unsigned cnt0[kFBins + 1];
  unsigned long long mass0[kFBins + 1];
  union {
    struct {  // sub-bin histogram of a crowded bin
      unsigned cnt1[kFBins];
      unsigned long long mass1[kFBins];
    } h;
    struct {
      unsigned keys[kFCap];  // gathered logits (order keys)
      unsigned rcnt[256];    // radix_cut's digit histogram over them (count, mass)
      unsigned long long rmass[256];
    } k;
    struct {  // deeper windows: the row's band counts, then capture counts
      unsigned tot[kDeep + 1];
      unsigned wc[kFWaves];
    } d;
    u32x4 stage[kFWaves][kStageVecs];  // deeper capture: each wave's staged vectors
  } u;
  FilterScratch sc;
};

// Whether a logit lies inside the capture window: y = z c - M > -kLevels (the
// same fma as every other use of y).
__device__ __forceinline__ bool in_window(float z, float c, float negM) {
  return fmaf(z, c, negM) > -static_cast<float>(kLevels);
}

__device__ __forceinline__ unsigned long long wave_incl_scan_u64(unsigned long long v, int lane) {
#pragma unroll
  for (int d = 1; d < kWave; d <<= 1) {
    const unsigned long long o = __shfl_up(v, d);
    if (lane >= d) v += o;
  }
  return v;
}

// Exclusive prefix of (a, b) over the workgroup's threads, with the totals.
__device__ __forceinline__ void wg_excl_scan2(unsigned long long &a, unsigned long long &b,
                                              unsigned long long &ta, unsigned long long &tb,
                                              unsigned long long *red) {
  const int lane = threadIdx.x & (kWave - 1), wave = threadIdx.x / kWave;
  const unsigned long long ia = wave_incl_scan_u64(a, lane), ib = wave_incl_scan_u64(b, lane);
  if (lane == kWave - 1) {
    red[wave] = ia;
    red[kFWaves + wave] = ib;
  }
  __syncthreads();
  unsigned long long pa = 0, pb = 0;
  ta = tb = 0;
#pragma unroll
  for (int w = 0; w < kFWaves; ++w) {
    const unsigned long long ra = red[w], rb = red[kFWaves + w];
    if (w < wave) {
      pa += ra;
      pb += rb;
    }
    ta += ra;
    tb += rb;
  }
  __syncthreads();
  a = pa + ia - a;
  b = pb + ib - b;
}

// First bin j of (cnt, mass)[0, n) whose inclusive prefix (of the counts, or of
// the masses when by_mass) reaches `target`, with the count and mass of the
// bins before it.  With no such bin (not reached for consistent sums) the last
// bin is returned.
__device__ int find_cross(const unsigned *cnt, const unsigned long long *mass, int n, bool by_mass,
                          unsigned long long target, unsigned long long &before_c,
                          unsigned long long &before_m, FilterScratch &sh) {
  const int per = (n + kFBlock - 1) / kFBlock;
  const int j0 = threadIdx.x * per, j1 = min(n, j0 + per);
  unsigned long long lc = 0, lm = 0;
  for (int j = j0; j < j1; ++j) {
    lc += cnt[j];
    lm += mass[j];
  }
  if (threadIdx.x == 0) sh.pick = -1;
  unsigned long long ec = lc, em = lm, tc, tm;
  wg_excl_scan2(ec, em, tc, tm, sh.red);
  const unsigned long long e = by_mass ? em : ec, l = by_mass ? lm : lc;
  if (j0 < j1 && e < target && target <= e + l) {  // exactly one thread
    unsigned long long rc = ec, rm = em;
    for (int j = j0; j < j1; ++j) {
      const unsigned long long v = by_mass ? mass[j] : cnt[j];
      if ((by_mass ? rm : rc) + v >= target) {
        sh.pick = j;
        sh.pick_c = rc;
        sh.pick_m = rm;
        break;
      }
      rc += cnt[j];
      rm += mass[j];
    }
  }
  __syncthreads();
  int j = sh.pick;
  if (j < 0) {
    j = n - 1;
    before_c = tc - cnt[j];
    before_m = tm - mass[j];
  } else {
    before_c = sh.pick_c;
    before_m = sh.pick_m;
  }
  __syncthreads();
  return j;
}

// Calls f(z) for every logit of the vectors [vb, ve) of a row (16-byte
// vectors; the row's last vector may be partial).  Whole vectors of an aligned
// row stream with U loads per thread per step, the next step's loads issued
// before the current step is processed (stream_chunk: every lane issues every
// load, indices clamped into the range, so the compiler waits for exactly the
// older step).  The partial tail, and every logit of an
// unaligned row, are read one by one.  keep(m) is asked with the largest logit
// m of each whole vector; a vector for which it answers false is skipped (for
// a test that is monotone in the logit this skips exactly the vectors none of
// whose logits would pass it).  Lanes leave the loops in decreasing order of
// their index: lane 0 of a wave is active whenever any lane of it is.
template <int DT, int BS, int U, typename K, typename F>
__device__ __forceinline__ void for_each_logit(const void *row, bool aligned, int V, long vb, long ve, K &&keep,
                                               F &&f) {
  constexpr int kV = Elem<DT>::kVec;
  const char *r = static_cast<const char *>(row);
  const long e_end = min(ve * kV, static_cast<long>(V));
  long e_tail = vb * kV;  // first logit left to the one-by-one loop
  if (aligned) {
    const int vw = static_cast<int>(min(ve, static_cast<long>(V) / kV));  // whole vectors in range
    const int tid = threadIdx.x;
    stream_chunk<DT, U, BS>(reinterpret_cast<const u32x4 *>(r), static_cast<int>(vb), vw, tid,
                            [&](const u32x4 *tile, int t0) {
#pragma unroll 1
                              for (int u = 0; u < U; ++u) {
                                if (t0 + u * BS + tid >= vw) break;
                                float x[kV];
                                widen_vec<DT>(tile[u], x);
                                float m = x[0];
#pragma unroll
                                for (int e = 1; e < kV; ++e) m = fmaxf(m, x[e]);
                                if (!keep(m)) continue;
#pragma unroll
                                for (int e = 0; e < kV; ++e) f(x[e]);
                              }
                            });
    e_tail = max(vb, static_cast<long>(vw)) * kV;
  }
  for (long e = e_tail + threadIdx.x; e < e_end; e += BS) f(load_one<DT>(row, e));
}

template <int DT, typename F>
__device__ __forceinline__ void for_each_logit(const void *row, bool aligned, int V, F &&f) {
  for_each_logit<DT, kFBlock, 8>(row, aligned, V, 0, (static_cast<long>(V) + Elem<DT>::kVec - 1) / Elem<DT>::kVec,
                                 [](float) { return true; }, static_cast<F &&>(f));
}

// The key interval of y bin j: every key in [lo, hi] maps to bin j and no
// other key does (the bin index is monotone in the key over the non-NaN keys).
__device__ __forceinline__ void bin_key_range(int j, float c, float negM, unsigned &lo, unsigned &hi) {
  const unsigned kmin = order_key(-INFINITY), kmax = order_key(INFINITY);
  unsigned a = kmin, z = kmax;  // smallest key with bin <= j
  while (a < z) {
    const unsigned mid = a + (z - a) / 2;
    if (ybin(key_value(mid), c, negM) <= j) z = mid;
    else a = mid + 1;
  }
  lo = a;
  a = kmin;
  z = kmax;  // largest key with bin >= j
  while (a < z) {
    const unsigned mid = a + (z - a + 1) / 2;
    if (ybin(key_value(mid), c, negM) >= j) a = mid;
    else z = mid - 1;
  }
  hi = a;
}

// Sorts keys[0, n) in descending order (bitonic, padded to a power of two
// with 0, which is below every non-NaN key).
__device__ void sort_keys_desc(unsigned *keys, int n) {
  const int tid = threadIdx.x;
  int N = 2;
  while (N < n) N <<= 1;
  for (int i = n + tid; i < N; i += kFBlock) keys[i] = 0u;
  __syncthreads();
  for (int size = 2; size <= N; size <<= 1) {
    for (int stride = size >> 1; stride > 0; stride >>= 1) {
      for (int i = tid; i < N / 2; i += kFBlock) {
        const int lo = 2 * i - (i & (stride - 1)), hi = lo + stride;
        const unsigned a = keys[lo], b = keys[hi];
        if (((lo & size) == 0) == (a < b)) {
          keys[lo] = b;
          keys[hi] = a;
        }
      }
      __syncthreads();
    }
  }
}

// Scan of sorted keys[0, n) (descending) that continue a prefix with count
// before_c and mass before_m: the first end of a group of equal keys whose
// inclusive count (by_mass false) or mass (by_mass true) reaches `target`.
// Returns its value; `kept` receives the inclusive mass there.
__device__ float scan_sorted(const unsigned *keys, int n, unsigned long long before_c,
                             unsigned long long before_m, bool by_mass, unsigned long long target,
                             float c, float negM, int fs, unsigned long long &kept, bool &found,
                             FilterScratch &sh) {
  constexpr int kPer = kFCap / kFBlock;
  const int tid = threadIdx.x;
  const int i0 = tid * kPer;
  unsigned long long m[kPer];
  unsigned long long lsum = 0;
#pragma unroll
  for (int q = 0; q < kPer; ++q) {
    m[q] = (i0 + q < n) ? fixed_mass(key_value(keys[i0 + q]), c, negM, fs) : 0ull;
    lsum += m[q];
  }
  unsigned long long ex = lsum, dummy = 0, tot, tdummy;
  wg_excl_scan2(ex, dummy, tot, tdummy, sh.red);
  if (tid == 0) sh.pick = 0x7fffffff;
  __syncthreads();
  unsigned long long run = before_m + ex;
  int mine = -1;
  unsigned long long mine_m = 0;
#pragma unroll
  for (int q = 0; q < kPer; ++q) {
    const int i = i0 + q;
    if (i < n) {
      run += m[q];
      const bool group_end = (i == n - 1) || keys[i + 1] != keys[i];
      const unsigned long long crit = by_mass ? run : before_c + static_cast<unsigned long long>(i) + 1;
      if (mine < 0 && group_end && crit >= target) {
        mine = i;
        mine_m = run;
      }
    }
  }
  if (mine >= 0) atomicMin(&sh.pick, mine);
  __syncthreads();
  const int pick = sh.pick;
  if (mine >= 0 && mine == pick) sh.res_m = mine_m;
  __syncthreads();
  float tau;
  found = pick != 0x7fffffff;
  if (!found) {  // not reached: keep all n
    tau = key_value(keys[n > 0 ? n - 1 : 0]);
    kept = before_m + tot;
  } else {
    tau = key_value(keys[pick]);
    kept = sh.res_m;
  }
  __syncthreads();
  return tau;
}

// The cut for one criterion over keys[0, n) in LDS (unsorted, n <= kFCap)
// that continue a prefix of before_c logits with mass before_m: the first end,
// from the top, of a group of equal keys whose inclusive count (by_mass false)
// or fixed-point mass (by_mass true), prefix included, reaches `target` --
// the definition scan_sorted applies to sorted keys -- found by an exact
// radix select.  One pass finds the keys' smallest and largest values and
// their totals; the bits above their highest differing bit are common to
// all.  Then one pass per 8-bit digit below that, from the top: an LDS
// histogram of (count, mass) over the digit of the keys that match the
// digits chosen so far, bins in descending digit order; one wave scans the 256
// bins and picks the bin where the running total crosses the target.  When
// every digit is chosen the keys left are one value: tau is that logit and
// kept the mass of every key >= it, prefix included.  Returns false (kept =
// the prefix plus the keys' total) when the target exceeds the total.  The
// keys of bf16 logits have their low 16 bits fixed by the sign (0 for keys
// >= 2^31, else all ones), so the digits stop at bit 16.
template <int DT>
__device__ bool radix_cut(const unsigned *keys, int n, unsigned long long before_c, unsigned long long before_m,
                          float c, float negM, int fs, bool by_mass, unsigned long long target, float &tau,
                          unsigned long long &kept, GeneralShared &sh) {
  constexpr int kLowBits = DT == SV_BF16 ? 16 : 0;
  const int tid = threadIdx.x, lane = tid & (kWave - 1), wave = tid / kWave;
  {  // smallest and largest key, count and mass of all the keys
    unsigned kmin = 0xffffffffu, kmax = 0u;
    unsigned long long tm = 0;
    for (int i = tid; i < n; i += kFBlock) {
      const unsigned key = keys[i];
      kmin = min(kmin, key);
      kmax = max(kmax, key);
      tm += fixed_mass(key_value(key), c, negM, fs);
    }
#pragma unroll
    for (int off = kWave / 2; off >= 1; off /= 2) {
      kmin = min(kmin, static_cast<unsigned>(__shfl_xor(static_cast<int>(kmin), off)));
      kmax = max(kmax, static_cast<unsigned>(__shfl_xor(static_cast<int>(kmax), off)));
      tm += __shfl_xor(tm, off);
    }
    if (lane == 0) {
      sh.sc.red[wave] = (static_cast<unsigned long long>(kmax) << 32) | kmin;
      sh.sc.red[kFWaves + wave] = tm;
    }
    __syncthreads();
    kmin = 0xffffffffu;
    kmax = 0u;
    tm = 0;
#pragma unroll
    for (int w = 0; w < kFWaves; ++w) {
      kmin = min(kmin, static_cast<unsigned>(sh.sc.red[w]));
      kmax = max(kmax, static_cast<unsigned>(sh.sc.red[w] >> 32));
      tm += sh.sc.red[kFWaves + w];
    }
    __syncthreads();
    const unsigned long long total = by_mass ? before_m + tm : before_c + static_cast<unsigned long long>(n);
    if (n == 0 || total < target) {  // not reached
      kept = before_m + tm;
      return false;
    }
    if (kmin == kmax) {  // one value
      tau = key_value(kmax);
      kept = before_m + tm;
      return true;
    }
    const int hb = 31 - __clz(static_cast<int>(kmin ^ kmax));  // highest differing bit
    unsigned hi_mask = hb >= 31 ? 0u : ~((2u << hb) - 1u);    // bits common to all keys
    unsigned hi_val = kmax & hi_mask;
    int shift = max(hb - 7, kLowBits);
    for (;;) {
      for (int j = tid; j < 256; j += kFBlock) {
        sh.u.k.rcnt[j] = 0;
        sh.u.k.rmass[j] = 0;
      }
      __syncthreads();
      for (int i = tid; i < n; i += kFBlock) {
        const unsigned key = keys[i];
        if ((key & hi_mask) == hi_val) {
          const int bin = 255 - static_cast<int>((key >> shift) & 255u);
          atomicAdd(&sh.u.k.rcnt[bin], 1u);
          atomicAdd(&sh.u.k.rmass[bin], fixed_mass(key_value(key), c, negM, fs));
        }
      }
      __syncthreads();
      if (tid < kWave) {  // lane L scans bins 4L .. 4L + 3
        unsigned long long bc[4], bm[4], lc = 0, lm = 0;
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          bc[q] = sh.u.k.rcnt[4 * lane + q];
          bm[q] = sh.u.k.rmass[4 * lane + q];
          lc += bc[q];
          lm += bm[q];
        }
        unsigned long long rc = wave_incl_scan_u64(lc, lane) - lc + before_c;
        unsigned long long rm = wave_incl_scan_u64(lm, lane) - lm + before_m;
        int mine = -1;
        unsigned long long mc = 0, mm = 0, mbin = 0;
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const unsigned long long before = by_mass ? rm : rc, here = by_mass ? bm[q] : bc[q];
          if (mine < 0 && before < target && target <= before + here) {
            mine = q;
            mc = rc;
            mm = rm;
            mbin = bm[q];
          }
          rc += bc[q];
          rm += bm[q];
        }
        if (mine >= 0) {  // exactly one lane: the running total reaches the target in the chosen keys
          sh.sc.pick = 4 * lane + mine;
          sh.sc.pick_c = mc;
          sh.sc.pick_m = mm;
          sh.sc.res_m = mbin;
        }
      }
      __syncthreads();
      const unsigned digit = 255u - static_cast<unsigned>(sh.sc.pick);
      before_c = sh.sc.pick_c;
      before_m = sh.sc.pick_m;
      const unsigned long long bin_m = sh.sc.res_m;
      __syncthreads();
      hi_val = (hi_val & ~(255u << shift)) | (digit << shift);
      hi_mask |= 255u << shift;
      if (shift == kLowBits) {
        const unsigned low = kLowBits == 0 ? 0u : ((hi_val & 0x80000000u) ? 0u : (1u << kLowBits) - 1u);
        tau = key_value(hi_val | low);
        kept = before_m + bin_m;
        return true;
      }
      shift = max(shift - 8, kLowBits);
    }
  }
}

// The threshold for one criterion: the first group of equal logits, from the
// top, whose inclusive count (by_mass false) or mass (by_mass true) reaches
// `target`.  Returns its value; `kept` receives the mass of all logits >= it.
template <int DT>
__device__ float resolve_cut(const void *row, bool aligned, int V, float c, float negM, int fs,
                             bool by_mass, unsigned long long target, unsigned long long &kept,
                             GeneralShared &sh) {
  const int tid = threadIdx.x;
  unsigned long long bc, bm;
  const int j = find_cross(sh.cnt0, sh.mass0, kFBins + 1, by_mass, target, bc, bm, sh.sc);
  unsigned count = sh.cnt0[j];
  if (tid == 0) bin_key_range(j, c, negM, sh.sc.klo, sh.sc.khi);
  __syncthreads();
  unsigned klo = sh.sc.klo, khi = sh.sc.khi;
  unsigned long long before_c = bc, before_m = bm;

  // split a crowded bin by the key until it fits the LDS buffer
  while (count > static_cast<unsigned>(kFCap)) {
    const unsigned range = khi - klo;
    const int shb = range >= static_cast<unsigned>(kFBins) ? (32 - __clz(range)) - 11 : 0;
    for (int i = tid; i < kFBins; i += kFBlock) {
      sh.u.h.cnt1[i] = 0;
      sh.u.h.mass1[i] = 0;
    }
    __syncthreads();
    for_each_logit<DT>(row, aligned, V, [&](float z) {
      const unsigned key = order_key(z);
      if (key >= klo && key <= khi) {
        const unsigned s = (khi - key) >> shb;
        atomicAdd(&sh.u.h.cnt1[s], 1u);
        const unsigned long long m = fixed_mass(z, c, negM, fs);
        if (m) atomicAdd(&sh.u.h.mass1[s], m);
      }
    });
    __syncthreads();
    const unsigned long long rel = target - (by_mass ? before_m : before_c);
    unsigned long long sc, sm;
    const int s = find_cross(sh.u.h.cnt1, sh.u.h.mass1, kFBins, by_mass, rel, sc, sm, sh.sc);
    before_c += sc;
    before_m += sm;
    count = sh.u.h.cnt1[s];
    const unsigned long long smass = sh.u.h.mass1[s];
    const long long top = static_cast<long long>(khi) - (static_cast<long long>(s) << shb);
    const long long bot = static_cast<long long>(khi) - (static_cast<long long>(s + 1) << shb) + 1;
    khi = static_cast<unsigned>(top);
    klo = bot > static_cast<long long>(klo) ? static_cast<unsigned>(bot) : klo;
    if (shb == 0) {  // one key: the whole group is one value
      kept = before_m + smass;
      __syncthreads();
      return key_value(khi);
    }
    __syncthreads();
  }

  // gather the bin's logits, sort them, scan
  if (tid == 0) sh.sc.nkeys = 0;
  __syncthreads();
  for_each_logit<DT>(row, aligned, V, [&](float z) {
    const unsigned key = order_key(z);
    if (key >= klo && key <= khi) {
      const unsigned slot = atomicAdd(&sh.sc.nkeys, 1u);
      if (slot < static_cast<unsigned>(kFCap)) sh.u.k.keys[slot] = key;
    }
  });
  __syncthreads();
  const int n = min(static_cast<int>(sh.sc.nkeys), kFCap);
  sort_keys_desc(sh.u.k.keys, n);
  bool found;
  return scan_sorted(sh.u.k.keys, n, before_c, before_m, by_mass, target, c, negM, fs, kept, found, sh.sc);
}

// Row selection shared by the filter kernels: request b's row r (target rows
// 0..gamma, then draft rows), or nullptr when the row is not filtered (greedy
// request, no active filter, or a row beyond the request's draft length).
template <int DT>
__device__ __forceinline__ const void *filtered_row(const void *target, const void *draft, const float *temps,
                                                    const int32_t *lens, const int32_t *topk, const float *topp,
                                                    int gamma, int V, int b, int r, float &T, int &k, float &p) {
  // the request's four parameters are fetched together (one round trip)
  T = temps[b];
  const int kr = topk ? topk[b] : 0;
  const float pr = topp ? topp[b] : 1.0f;
  const int g = request_len(lens, gamma, b);
  const bool filters = filter_params(kr, pr, V, k, p);
  if (!(T > 0.0f) || !filters) return nullptr;
  const bool is_target = r <= gamma;
  const int i = is_target ? r : r - gamma - 1;
  if (is_target ? i > g : i >= g) return nullptr;
  return is_target ? static_cast<const void *>(static_cast<const char *>(target) +
                                               (static_cast<long>(b) * (gamma + 1) + i) * V * Elem<DT>::kBytes)
                   : static_cast<const void *>(static_cast<const char *>(draft) +
                                               (static_cast<long>(b) * gamma + i) * V * Elem<DT>::kBytes);
}

// The row's M (and K1's row sum s), merged in chunk order as K2 merges them.
__device__ __forceinline__ void row_scale(const Partial *part, long slot, int NS, int &M, double &s) {
  M = kEmptyM;
  s = 0.0;
  float mx = -INFINITY;
  for (int j0 = 0; j0 < NS; j0 += kK2Batch) {  // partials fetched kK2Batch at a time
    Partial buf[kK2Batch];
#pragma unroll
    for (int u = 0; u < kK2Batch; ++u)
      if (j0 + u < NS) buf[u] = part[slot * NS + j0 + u];
#pragma unroll
    for (int u = 0; u < kK2Batch; ++u)
      if (j0 + u < NS) merge_sm(M, s, mx, buf[u].mi, buf[u].s, buf[u].mx);
  }
}

// FG: one chunk of a row (K1's chunking).  Every logit with y > -kLevels is a
// candidate.  Each wave gathers its candidates in its own LDS region (slots
// from a ballot: no atomics), then reserves its range of the row's list with
// one atomic and copies them out.  A wave that finds more than kWaveCap
// candidates pushes the row's count past kGCap (the general path).
constexpr int kWaveCap = 2048;

template <int DT>
__global__ __launch_bounds__(kLBlock) void k_filter_capture(
    const void *__restrict__ target, const void *__restrict__ draft, const float *__restrict__ temps,
    const int32_t *__restrict__ lens, const int32_t *__restrict__ topk, const float *__restrict__ topp,
    int gamma, int V, int NS, int chunk_vecs, const Partial *__restrict__ part, FilterWork fw) {
  constexpr int kV = Elem<DT>::kVec;
  constexpr int U = 8;
  const int rows = 2 * gamma + 1;
  const long slot = blockIdx.x / NS;
  const int j = static_cast<int>(blockIdx.x - slot * NS);
  const int b = static_cast<int>(slot / rows), r = static_cast<int>(slot - static_cast<long>(b) * rows);
  float T, p;
  int k;
  const void *row = filtered_row<DT>(target, draft, temps, lens, topk, topp, gamma, V, b, r, T, k, p);
  if (!row) return;  // uniform per workgroup
  const bool aligned = (reinterpret_cast<uintptr_t>(row) & 15u) == 0;
  int M;
  double s;
  row_scale(part, slot, NS, M, s);
  const float c = temp_scale(T), negM = -static_cast<float>(M);
  const int tid = threadIdx.x, lane = tid & (kWave - 1), wave = tid / kWave;
  __shared__ unsigned wbuf[kLBlock / kWave][kWaveCap];
  unsigned wcount = 0;  // the same in every lane of the wave
  const unsigned long long lt = (1ull << lane) - 1ull;
  auto offer = [&](float z) {  // called by every lane of the wave together
    const bool in = in_window(z, c, negM);
    const unsigned long long mask = __ballot(in);
    if (in) {
      const unsigned q = wcount + static_cast<unsigned>(__popcll(mask & lt));
      if (q < static_cast<unsigned>(kWaveCap)) wbuf[wave][q] = order_key(z);
    }
    wcount += static_cast<unsigned>(__popcll(mask));
  };
  // Vectors that hold a candidate are rare on most rows, so a lane whose
  // vector's maximum passes the window test copies the raw vector into the
  // wave's staging area (one 16-byte LDS store), and the wave offers the
  // staged logits together, 64 at a time, once the area is half full: one
  // ballot round per 64 staged logits instead of one per logit of every
  // vector round with a candidate somewhere in the wave.
  __shared__ u32x4 stage[kLBlock / kWave][kStageVecs];
  unsigned nst = 0;  // vectors staged by the wave (the same in every lane)
  auto flush = [&]() {
    __builtin_amdgcn_wave_barrier();  // the stores above come first
    const unsigned n = nst * static_cast<unsigned>(kV);
    for (unsigned i0 = 0; i0 < n; i0 += kWave) {
      const unsigned i = i0 + static_cast<unsigned>(lane);
      float z = -INFINITY;
      if (i < n) {
        if constexpr (DT == SV_F32) z = reinterpret_cast<const float *>(stage[wave])[i];
        else z = __uint_as_float(static_cast<uint32_t>(reinterpret_cast<const uint16_t *>(stage[wave])[i]) << 16);
      }
      offer(z);
    }
    __builtin_amdgcn_wave_barrier();  // the loads above complete before the area is reused
    nst = 0;
  };
  const char *rb = static_cast<const char *>(row);
  const long nvec = (static_cast<long>(V) + kV - 1) / kV;
  const long vb = static_cast<long>(j) * chunk_vecs, ve = min(vb + chunk_vecs, nvec);
  const long vw = aligned ? min(ve, static_cast<long>(V) / kV) : vb;  // whole 16-byte vectors
  // whole vectors (K1's streaming: non-temporal loads, the next tile in flight
  // while this one is examined): the same trip count in every lane, and
  // out-of-range vectors read as -inf
  stream_chunk<DT, U, kLBlock>(reinterpret_cast<const u32x4 *>(rb), static_cast<int>(vb), static_cast<int>(vw), tid,
                               [&](const u32x4 *tile, int) {
#pragma unroll
                                 for (int u = 0; u < U; ++u) {
                                   float x[kV];
                                   widen_vec<DT>(tile[u], x);
                                   float m = x[0];
#pragma unroll
                                   for (int e = 1; e < kV; ++e) m = fmaxf(m, x[e]);
                                   const bool hit = in_window(m, c, negM);
                                   const unsigned long long F = __ballot(hit);
                                   if (!F) continue;  // no lane of the wave has a candidate
                                   if (hit) stage[wave][nst + static_cast<unsigned>(__popcll(F & lt))] = tile[u];
                                   nst += static_cast<unsigned>(__popcll(F));
                                   if (nst > kStageVecs - kWave) flush();
                                 }
                               });
  if (nst) flush();
  // the rest one by one (a partial last vector, or a row that is not aligned)
  const long e0 = max(vb, vw) * kV, e1 = min(ve * kV, static_cast<long>(V));
  for (long eb = e0; eb < e1; eb += kLBlock) {
    const long e = eb + tid;
    offer(e < e1 ? load_one<DT>(row, e) : -INFINITY);
  }
  // reserve the wave's range of the row's list and copy it out
  unsigned *cnt = fw.ncand + slot;
  unsigned *cand = fw.cand + slot * kGCap;
  unsigned base = 0;
  if (lane == 0 && wcount > 0)
    base = atomicAdd(cnt, wcount <= static_cast<unsigned>(kWaveCap) ? wcount : static_cast<unsigned>(kGCap) + 1u);
  base = static_cast<unsigned>(__shfl(static_cast<int>(base), 0));
  if (wcount <= static_cast<unsigned>(kWaveCap)) {
    for (unsigned i = lane; i < wcount; i += kWave)
      if (base + i < static_cast<unsigned>(kGCap)) cand[base + i] = wbuf[wave][i];
  }
}

// The cut for one criterion from a row's candidate list, whose histogram is in
// sh.cnt0 / sh.mass0: the bin that reaches the target, whose candidates are
// gathered and resolved by radix_cut from the prefix above it.  ok is false
// when that bin holds more than kFCap candidates or the target is not reached.
template <int DT>
__device__ float list_cut(const unsigned *cand, int n, float c, float negM, int fs, bool by_mass,
                          unsigned long long target, unsigned long long &kept, bool &ok, GeneralShared &sh) {
  const int tid = threadIdx.x;
  unsigned long long bc, bm;
  const int jb = find_cross(sh.cnt0, sh.mass0, kFBins + 1, by_mass, target, bc, bm, sh.sc);
  if (sh.cnt0[jb] > static_cast<unsigned>(kFCap)) {  // uniform
    ok = false;
    return -INFINITY;
  }
  if (tid == 0) sh.sc.nkeys = 0;
  __syncthreads();
  for (int i = tid; i < n; i += kFBlock) {
    const unsigned key = cand[i];
    if (ybin(key_value(key), c, negM) == jb) {
      const unsigned q = atomicAdd(&sh.sc.nkeys, 1u);
      if (q < static_cast<unsigned>(kFCap)) sh.u.k.keys[q] = key;
    }
  }
  __syncthreads();
  const int m = min(static_cast<int>(sh.sc.nkeys), kFCap);
  float tau = -INFINITY;
  ok = radix_cut<DT>(sh.u.k.keys, m, bc, bm, c, negM, fs, by_mass, target, tau, kept, sh);
  return tau;
}

// The top-p target in fixed point: top_p of the top-k mass (k > 0), or of
// the row's mass (K1's sum s, in the same units), at least 1.
__device__ __forceinline__ unsigned long long p_target(int k, float p, unsigned long long topk_mass, double s,
                                                       int fs) {
  const double base = k > 0 ? static_cast<double>(topk_mass) : ldexp(s, fs);
  double t = ceil(static_cast<double>(p) * base);
  if (t < 1.0) t = 1.0;
  return static_cast<unsigned long long>(t);
}

// The cut of a row from a list that holds every logit above some floor y = -L
// (L <= 64): the count criterion (top-k), then the mass criterion (top-p of
// the top-k mass, or of K1's row sum s).  Returns false when the list cannot
// decide the cut; short_list is then true when the k-th logit or the crossing
// lies below the floor.  list_mass receives the list's fixed-point mass.
//   direct     at most kFCap logits: copied into LDS, and each criterion
//              resolved by radix_cut over all of them;
//   histogram  more: an exact (count, fixed-point mass) histogram of the list
//              over 1/32-order bins finds the bin of each crossing, whose
//              logits are gathered and resolved by radix_cut from the prefix
//              above it (list_cut).
// Both take the same sums of the same integers, so they give the same cut.
template <int DT>
__device__ bool list_resolve(const unsigned *cand, int n, float c, float negM, int fs, int k, float p, double s,
                             float &tau, unsigned long long &kept, unsigned long long &list_mass, bool &short_list,
                             GeneralShared &sh) {
  const int tid = threadIdx.x;
  tau = -INFINITY;
  kept = 0;
  short_list = false;
  if (n <= kFCap) {  // uniform: the direct path
    if (k > n) {  // the k-th logit lies below the floor
      short_list = true;
      list_mass = 0;
      return false;
    }
    for (int i = tid; i < n; i += kFBlock) sh.u.k.keys[i] = cand[i];
    __syncthreads();
    bool ok = true;
    if (k > 0)
      radix_cut<DT>(sh.u.k.keys, n, 0ull, 0ull, c, negM, fs, false, static_cast<unsigned long long>(k), tau, kept, sh);
    list_mass = 0;  // not needed by the callers on this path
    if (p < 1.0f) {
      float tau_p;
      unsigned long long kept_p;
      if (!radix_cut<DT>(sh.u.k.keys, n, 0ull, 0ull, c, negM, fs, true, p_target(k, p, kept, s, fs), tau_p, kept_p,
                         sh)) {
        ok = false;  // the crossing lies below the floor
        short_list = true;
      } else if (tau_p > tau) {
        tau = tau_p;
        kept = kept_p;
      }
    }
    __syncthreads();
    return ok;
  }
  for (int jb = tid; jb <= kFBins; jb += kFBlock) {
    sh.cnt0[jb] = 0;
    sh.mass0[jb] = 0;
  }
  __syncthreads();
  for (int i = tid; i < n; i += kFBlock) {
    const float z = key_value(cand[i]);
    const int jb = ybin(z, c, negM);
    atomicAdd(&sh.cnt0[jb], 1u);
    const unsigned long long m = fixed_mass(z, c, negM, fs);
    if (m) atomicAdd(&sh.mass0[jb], m);
  }
  __syncthreads();
  unsigned long long total_m = 0;
  {
    unsigned long long lm = 0, lc = 0, tc;
    for (int jb = tid; jb <= kFBins; jb += kFBlock) lm += sh.mass0[jb];
    wg_excl_scan2(lm, lc, total_m, tc, sh.sc.red);
  }
  list_mass = total_m;
  bool ok = true;
  if (k > 0) {
    if (k > n) {  // the k-th logit lies below the floor
      ok = false;
      short_list = true;
    } else {
      tau = list_cut<DT>(cand, n, c, negM, fs, false, static_cast<unsigned long long>(k), kept, ok, sh);
    }
  }
  if (ok && p < 1.0f) {
    const unsigned long long tgt = p_target(k, p, kept, s, fs);
    if (total_m < tgt) {  // the crossing lies below the floor
      ok = false;
      short_list = true;
    } else {
      unsigned long long kept_p;
      const float tau_p = list_cut<DT>(cand, n, c, negM, fs, true, tgt, kept_p, ok, sh);
      if (ok && tau_p > tau) {
        tau = tau_p;
        kept = kept_p;
      }
    }
  }
  __syncthreads();
  return ok;
}

__device__ __forceinline__ int deep_level(int j) { return kLevels + 2 * (j + 1); }

// Per-thread counts of the logits of vectors [vb, vw) (whole 16-byte vectors of
// an aligned row, streamed as in K1) and elements [e0, e1) (one by one) in the
// bands between the deeper floors: band b holds the logits with
// floor(-y/2 - 8) = b, clamped to [0, kDeep] (b = 0: above y = -18, the first
// deeper floor; b = kDeep: at or below y = -40), so that the count above floor
// j (y > -(18 + 2 j)) is the sum of bands 0..j.  -y/2 - 8 is exact for
// y > -64, so each band test agrees with the compare y > -L.  A logit costs
// a handful of operations: its band's one-hot nibble is added to a 64-bit
// word, which is spread into byte counters once per vector and into 32-bit
// counters once per tile.
template <int DT, int BS, int U>
__device__ __forceinline__ void count_bands(const void *row, int vb, int vw, long e0, long e1, float c, float negM,
                                            unsigned *cnt) {
  constexpr int kV = Elem<DT>::kVec;
  constexpr unsigned long long kLow = 0x0F0F0F0F0F0F0F0Full;
  const int tid = threadIdx.x;
#pragma unroll
  for (int j = 0; j <= kDeep; ++j) cnt[j] = 0;
  auto nibble = [&](float z) {
    const float q = fmaf(fmaf(z, c, negM), -0.5f, -8.0f);
    const int b = static_cast<int>(fminf(fmaxf(floorf(q), 0.0f), static_cast<float>(kDeep)));
    return 1ull << (4 * b);
  };
  // even bands in the bytes of ev, odd bands in the bytes of od
  auto spread = [&](unsigned long long nib, unsigned long long &ev, unsigned long long &od) {
    ev += nib & kLow;
    od += (nib >> 4) & kLow;
  };
  auto flush = [&](unsigned long long ev, unsigned long long od) {
#pragma unroll
    for (int j = 0; j <= kDeep; ++j)
      cnt[j] += static_cast<unsigned>(((j & 1) ? od : ev) >> (8 * (j >> 1))) & 0xFFu;
  };
  stream_chunk<DT, U, BS>(reinterpret_cast<const u32x4 *>(row), vb, vw, tid, [&](const u32x4 *tile, int) {
    unsigned long long ev = 0, od = 0;  // at most U * kV <= 64 per byte
#pragma unroll
    for (int u = 0; u < U; ++u) {
      float x[kV];
      widen_vec<DT>(tile[u], x);
      unsigned long long nib = 0;  // at most kV <= 8 per nibble
#pragma unroll
      for (int e = 0; e < kV; ++e) nib += nibble(x[e]);
      spread(nib, ev, od);
    }
    flush(ev, od);
  });
  for (long eb = e0; eb < e1; eb += BS) {
    const long e = eb + tid;
    if (e < e1) {
      unsigned long long ev = 0, od = 0;
      spread(nibble(load_one<DT>(row, e)), ev, od);
      flush(ev, od);
    }
  }
}

// The floor for the deeper list from the row's band counts band[0..kDeep]:
// the level count L of the shallowest floor whose logits include the k-th
// largest, provided that floor holds at most kFCap logits; 0 otherwise.
__device__ __forceinline__ int choose_floor(const unsigned *band, int k) {
  unsigned C = 0;  // logits above floor j
  for (int j = 0; j < kDeep; ++j) {
    C += band[j];
    if (C >= static_cast<unsigned>(k)) return C <= static_cast<unsigned>(kFCap) ? deep_level(j) : 0;
  }
  return 0;
}

// Second pass: every logit with y > -L goes to the row's list.  Each wave
// fills its own part of the list (slots from a ballot, a scalar count; the
// vectors that can hold such a logit are first staged in LDS and offered 64
// logits at a time), then the parts are packed to the front of the list
// through LDS.  Returns the list's length, or kGCap + 1 when a wave's part
// overflowed.
template <int DT>
__device__ unsigned deep_capture(const void *row, bool aligned, int V, float c, float negM, int L,
                                 unsigned *cand, GeneralShared &sh) {
  constexpr unsigned kPart = kGCap / kFWaves;
  const int tid = threadIdx.x, lane = tid & (kWave - 1), wave = tid / kWave;
  const float floor_y = -static_cast<float>(L);
  const unsigned long long lt = (1ull << lane) - 1ull;
  unsigned *part = cand + wave * kPart;
  unsigned wcount = 0;  // the same in every lane of the wave
  auto offer = [&](float z) {  // called by every lane of the wave together
    const bool in = fmaf(z, c, negM) > floor_y;
    const unsigned long long mask = __ballot(in);
    if (in) {
      const unsigned q = wcount + static_cast<unsigned>(__popcll(mask & lt));
      if (q < kPart) part[q] = order_key(z);
    }
    wcount += static_cast<unsigned>(__popcll(mask));
  };
  // as in the capture kernel: a vector whose maximum passes the floor is staged
  // in LDS, and the wave offers the staged logits 64 per ballot round
  constexpr int kV = Elem<DT>::kVec;
  unsigned nst = 0;
  auto flush = [&]() {
    __builtin_amdgcn_wave_barrier();
    const unsigned n = nst * static_cast<unsigned>(kV);
    for (unsigned i0 = 0; i0 < n; i0 += kWave) {
      const unsigned i = i0 + static_cast<unsigned>(lane);
      float z = -INFINITY;
      if (i < n) {
        if constexpr (DT == SV_F32) z = reinterpret_cast<const float *>(sh.u.stage[wave])[i];
        else z = __uint_as_float(static_cast<uint32_t>(reinterpret_cast<const uint16_t *>(sh.u.stage[wave])[i]) << 16);
      }
      offer(z);
    }
    __builtin_amdgcn_wave_barrier();
    nst = 0;
  };
  const int vw = aligned ? V / kV : 0;  // whole 16-byte vectors
  stream_chunk<DT, 8, kFBlock>(reinterpret_cast<const u32x4 *>(row), 0, vw, tid, [&](const u32x4 *tile, int) {
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      float x[kV];
      widen_vec<DT>(tile[u], x);
      float m = x[0];
#pragma unroll
      for (int e = 1; e < kV; ++e) m = fmaxf(m, x[e]);
      const bool hit = fmaf(m, c, negM) > floor_y;  // fma is monotonic in z for c > 0
      const unsigned long long F = __ballot(hit);
      if (!F) continue;
      if (hit) sh.u.stage[wave][nst + static_cast<unsigned>(__popcll(F & lt))] = tile[u];
      nst += static_cast<unsigned>(__popcll(F));
      if (nst > kStageVecs - kWave) flush();
    }
  });
  if (nst) flush();
  // the rest one by one (a partial last vector, or a row that is not aligned)
  for (long eb = static_cast<long>(vw) * kV; eb < V; eb += kFBlock) {
    const long e = eb + tid;
    offer(e < V ? load_one<DT>(row, e) : -INFINITY);
  }
  __syncthreads();  // every wave is done with its staging area, which wc overlaps
  if (lane == 0) sh.u.d.wc[wave] = wcount;
  __syncthreads();
  unsigned total = 0, before = 0;
  bool over = false;
  for (int w = 0; w < kFWaves; ++w) {
    const unsigned nw = sh.u.d.wc[w];
    if (w < wave) before += nw;
    total += nw;
    over = over || nw > kPart;
  }
  __syncthreads();
  if (over || total > static_cast<unsigned>(kFCap)) return static_cast<unsigned>(kGCap) + 1u;
  for (unsigned i = lane; i < wcount; i += kWave) sh.u.k.keys[before + i] = part[i];
  __syncthreads();
  for (unsigned i = tid; i < total; i += kFBlock) cand[i] = sh.u.k.keys[i];
  __syncthreads();
  return total;
}

// Row setup shared by the filter kernels after FG: the row (nullptr when it
// is not filtered), its alignment, M and K1's row sum.
struct FilterRow {
  const void *row;
  bool aligned;
  int k;
  float p, c, negM;
  double s;
};

template <int DT>
__device__ __forceinline__ FilterRow filter_row_setup(const void *target, const void *draft, const float *temps,
                                                      const int32_t *lens, const int32_t *topk, const float *topp,
                                                      int gamma, int V, int NS, const Partial *part, long slot) {
  const int rows = 2 * gamma + 1;
  const int b = static_cast<int>(slot / rows), r = static_cast<int>(slot - static_cast<long>(b) * rows);
  FilterRow fr;
  float T;
  fr.row = filtered_row<DT>(target, draft, temps, lens, topk, topp, gamma, V, b, r, T, fr.k, fr.p);
  if (!fr.row) return fr;
  fr.aligned = (reinterpret_cast<uintptr_t>(fr.row) & 15u) == 0;
  int M;
  row_scale(part, slot, NS, M, fr.s);
  fr.c = temp_scale(T);
  fr.negM = -static_cast<float>(M);
  return fr;
}

// FilterStats.pad after FC, for every row: 0 resolved (or not filtered), 1 pending for the
// general path (FE).
enum { kFResolved = 0, kFGeneral = 1 };

__device__ __forceinline__ void store_filter_stats(FilterStats *fst, long slot, unsigned long long kept, int fs,
                                                   float tau, int state) {
  if (threadIdx.x == 0) {
    FilterStats f;
    f.s_kept = ldexp(static_cast<double>(kept), -fs);
    f.tau = tau;
    f.pad = state;
    fst[slot] = f;
  }
}

// Whether top-k row `slot` captured fewer logits than k (its k-th logit lies
// below the capture window): FD counts it, FC takes a deeper list.
__device__ __forceinline__ bool needs_deeper(int k, const FilterWork &fw, long slot) {
  return k > 0 && fw.ncand[slot] < static_cast<unsigned>(k);
}

// FD: K1's chunks of every top-k row whose k-th logit lies below the capture
// window (fewer than k logits captured): each chunk's counts above the floors.
template <int DT>
__global__ __launch_bounds__(kLBlock) void k_filter_deep_count(
    const void *__restrict__ target, const void *__restrict__ draft, const float *__restrict__ temps,
    const int32_t *__restrict__ lens, const int32_t *__restrict__ topk, const float *__restrict__ topp,
    int gamma, int V, int NS, int chunk_vecs, const Partial *__restrict__ part, FilterWork fw) {
  constexpr int kV = Elem<DT>::kVec;
  const long slot = blockIdx.x / NS;
  const int j = static_cast<int>(blockIdx.x - slot * NS);
  {  // most rows need no deeper count: decide that from top_k and the captured
     // count alone (one round trip) before the rest of the row's set-up
    const int b = static_cast<int>(slot / (2 * gamma + 1));
    const int kr = topk[b];
    const unsigned nc = fw.ncand[slot];
    if (!(kr > 0 && kr < V && nc < static_cast<unsigned>(kr))) return;  // uniform per workgroup
  }
  const FilterRow fr = filter_row_setup<DT>(target, draft, temps, lens, topk, topp, gamma, V, NS, part, slot);
  if (!fr.row || !needs_deeper(fr.k, fw, slot)) return;  // uniform per workgroup
  // the chunk's whole vectors, then its remaining elements (the capture kernel's split)
  const long nvec = (static_cast<long>(V) + kV - 1) / kV;
  const long vb = static_cast<long>(j) * chunk_vecs, ve = min(vb + chunk_vecs, nvec);
  const long vw = fr.aligned ? min(ve, static_cast<long>(V) / kV) : vb;
  const long e0 = max(vb, vw) * kV, e1 = min(ve * kV, static_cast<long>(V));
  unsigned cnt[kDeep + 1];
  count_bands<DT, kLBlock, 8>(fr.row, static_cast<int>(vb), static_cast<int>(vw), e0, e1, fr.c, fr.negM, cnt);
  __shared__ unsigned wcnt[kLBlock / kWave][kDeep + 1];
  const int lane = threadIdx.x & (kWave - 1), wave = threadIdx.x / kWave;
#pragma unroll
  for (int f = 0; f <= kDeep; ++f) {
#pragma unroll
    for (int off = kWave / 2; off >= 1; off /= 2)
      cnt[f] += static_cast<unsigned>(__shfl_xor(static_cast<int>(cnt[f]), off));
  }
  if (lane == 0) {
#pragma unroll
    for (int f = 0; f <= kDeep; ++f) wcnt[wave][f] = cnt[f];
  }
  __syncthreads();
  if (threadIdx.x <= kDeep) {
    unsigned t = 0;
    for (int w = 0; w < kLBlock / kWave; ++w) t += wcnt[w][threadIdx.x];
    fw.dcount[(slot * NS + j) * (kDeep + 1) + threadIdx.x] = t;
  }
}

// FC: one workgroup per row.  Resolves the cut from the row's captured list,
// or, for a top-k row whose k-th logit lies below the window, from a deeper
// list: the floor from FD's counts, a capture pass, the list resolve.  Rows it
// cannot resolve are left for FE.
template <int DT>
__global__ __launch_bounds__(kFBlock) void k_filter_resolve(
    const void *__restrict__ target, const void *__restrict__ draft, const float *__restrict__ temps,
    const int32_t *__restrict__ lens, const int32_t *__restrict__ topk, const float *__restrict__ topp,
    int gamma, int V, int NS, int fs, const Partial *__restrict__ part, FilterWork fw,
    FilterStats *__restrict__ fst) {
  const long slot = blockIdx.x;
  const FilterRow fr = filter_row_setup<DT>(target, draft, temps, lens, topk, topp, gamma, V, NS, part, slot);
  if (!fr.row) {  // uniform per workgroup: marked resolved, so that FE needs one load to skip it
    store_filter_stats(fst, slot, 0ull, fs, -INFINITY, kFResolved);
    return;
  }
  __shared__ GeneralShared sh;
  float tau = -INFINITY;
  unsigned long long kept = 0, list_mass;
  bool done = false, short_list;
  unsigned *cand = fw.cand + slot * kGCap;
  unsigned n = fw.ncand[slot];
  if (needs_deeper(fr.k, fw, slot)) {
    if (threadIdx.x <= kDeep) {
      unsigned t = 0;
      for (int j = 0; j < NS; ++j) t += fw.dcount[(slot * NS + j) * (kDeep + 1) + threadIdx.x];
      sh.u.d.tot[threadIdx.x] = t;
    }
    __syncthreads();
    const int L = choose_floor(sh.u.d.tot, fr.k);
    __syncthreads();
    n = L > 0 ? deep_capture<DT>(fr.row, fr.aligned, V, fr.c, fr.negM, L, cand, sh) : kGCap + 1u;
  }
  if (n <= static_cast<unsigned>(kGCap))
    done = list_resolve<DT>(cand, static_cast<int>(n), fr.c, fr.negM, fs, fr.k, fr.p, fr.s, tau, kept, list_mass,
                        short_list, sh);
  store_filter_stats(fst, slot, kept, fs, tau, done ? kFResolved : kFGeneral);
}

// FE: one workgroup per row still pending: the general path.
template <int DT>
__global__ __launch_bounds__(kFBlock) void k_filter_general(
    const void *__restrict__ target, const void *__restrict__ draft, const float *__restrict__ temps,
    const int32_t *__restrict__ lens, const int32_t *__restrict__ topk, const float *__restrict__ topp,
    int gamma, int V, int NS, int fs, const Partial *__restrict__ part, FilterStats *__restrict__ fst) {
  const long slot = blockIdx.x;
  if (fst[slot].pad != kFGeneral) return;  // uniform; FC stores every row's state
  const FilterRow fr = filter_row_setup<DT>(target, draft, temps, lens, topk, topp, gamma, V, NS, part, slot);
  const void *row = fr.row;
  const bool aligned = fr.aligned;
  const int k = fr.k;
  const float p = fr.p, c = fr.c, negM = fr.negM;
  __shared__ GeneralShared sh;
  const int tid = threadIdx.x;
  for (int jb = tid; jb <= kFBins; jb += kFBlock) {
    sh.cnt0[jb] = 0;
    sh.mass0[jb] = 0;
  }
  __syncthreads();
  for_each_logit<DT>(row, aligned, V, [&](float z) {
    const int jb = ybin(z, c, negM);
    atomicAdd(&sh.cnt0[jb], 1u);
    const unsigned long long m = fixed_mass(z, c, negM, fs);
    if (m) atomicAdd(&sh.mass0[jb], m);
  });
  __syncthreads();
  unsigned long long total = 0;
  {
    unsigned long long lm = 0, lc = 0, tc;
    for (int jb = tid; jb <= kFBins; jb += kFBlock) lm += sh.mass0[jb];
    wg_excl_scan2(lm, lc, total, tc, sh.sc.red);
  }
  float tau = -INFINITY;
  unsigned long long kept = total;
  if (k > 0)
    tau = resolve_cut<DT>(row, aligned, V, c, negM, fs, false, static_cast<unsigned long long>(k), kept, sh);
  if (p < 1.0f) {
    double t = ceil(static_cast<double>(p) * static_cast<double>(kept));
    if (t < 1.0) t = 1.0;
    unsigned long long tgt = static_cast<unsigned long long>(t);
    if (tgt > kept) tgt = kept;
    unsigned long long kept_p;
    const float tau_p = resolve_cut<DT>(row, aligned, V, c, negM, fs, true, tgt, kept_p, sh);
    if (tau_p > tau) {
      tau = tau_p;
      kept = kept_p;
    }
  }
  store_filter_stats(fst, slot, kept, fs, tau, kFResolved);
}

// ================================================================== tree verification
// A tree of drafts per request: node n (n < N_b) has parent[n] in [-1, n)
// (-1: the verified prefix) and token[n]; position 0 is the prefix and
// position n + 1 is node n.  Target row j and draft row j are the target and
// the draft distribution at position j (the layout of the linear call with
// gamma = max_nodes, so K1 computes every row's statistics unchanged).
//
// The pages draw such trees but verify them with a lossy threshold; the rule
// here is a reading that stays lossless: the children of a position are
// independent draws from its draft distribution q, tested in node order, the
// first against p and each later one against max(0, p_cur - q) / sum, the
// modified distribution of the previous rejection.  With p_j the target after
// j rejections, p_j = max(0, p - c_j q) / Z_j where c_0 = 0, Z_0 = 1 and
// c_{j+1} = c_j + Z_j (the recursion unrolled), so one pass over the row pair
// per rejection gives Z_{j+1}.  An accepted child moves to its position; if
// every child is rejected, or there is none, the token is drawn from p_j by
// the inverse CDF with u_sample.  T == 0 follows the first child equal to the
// target arg-max.
//
// k_tree_walk: NW 256-thread workgroups per request walk its tree together.
// Every workgroup takes the same decisions (the row statistics, from K1's
// partials or computed by the team for the positions it visits, the acceptance
// ratio in fp64 from the two gathered logits, all merged and summed in a fixed
// order); each rejection costs one pass over the position's two rows, shared
// out as 2048-token sub-chunks over the request's NW x 4 waves.  Each
// sub-chunk mass (and each wave's statistics) goes out with the exchange
// number in 64-bit device-scope atomic stores into per-request arrays (two
// copies each, alternating between exchanges, zeroed before the walk by K1 or
// by a clear); each workgroup polls the words until all carry the exchange
// number and merges them in the same order, so the results are the same
// everywhere.  Workgroup 0 writes the outputs; the final token is drawn by the
// wave that holds its sub-chunk, else by workgroup 0.  With NW = 1 (large
// batches) the exchanged values stay in LDS.
// The walk's workgroup barrier orders LDS only.  Its threads share nothing
// else through memory (the team's words are device-scope atomics), and a full
// barrier would wait for every global load the wave has in flight, such as the
// row slices requested for the passes to come.
__device__ __forceinline__ void tree_barrier() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

// s_waitcnt vmcnt(0) (expcnt and lgkmcnt left at their maxima, 7 and 15)
constexpr int kWaitVmcnt0 = 0x0F70;

constexpr int kTBlock = 256;
// Trees of at least this many nodes take their row statistics from the walk
// itself (only the positions it visits: a path of a wide tree is a small share
// of its rows); smaller trees take them from K1 over every row.  Per call on
// trees of V = 128256 bf16 (B = 8 unless stated; K1 then walk / walk alone):
// width 4 depth 3 (84 nodes) 82.3 / 40.0 us, B = 32 252 / 75.6, width 2 depth
// 4 (30) 58.2 / 40.9, width 2 depth 3 (14) 44.2 / 40.6, width 3 depth 2 (12)
// 38.4 / 33.0, a chain of 6 52.3 / 54.6.
constexpr int kTreeOnDemandNodes = 8;
constexpr int kTWaves = kTBlock / kWave;
constexpr int kTMaxSub = SV_TREE_MAX_V / kSub;
constexpr int kTMaxNS = 2 * kWave;
constexpr int kTMaxNodesPerLane = SV_TREE_MAX_NODES / kWave;  // children of a position per lane of one wave  // chunks per row: at most 128 (V <= 2^20 fp32 is 128 K1 tiles)
static_assert(SV_TREE_MAX_NODES <= kTBlock, "one thread per node in the child compaction");

struct TreeShared {
  int parent[SV_TREE_MAX_NODES];
  int token[SV_TREE_MAX_NODES];
  int child[SV_TREE_MAX_NODES];    // children of the current position, in node order
  int childp[SV_TREE_MAX_NODES];   // children of the prefetched position
  float czp[SV_TREE_MAX_NODES];    // their target and draft logits, and uniforms
  float czq[SV_TREE_MAX_NODES];
  float cu[SV_TREE_MAX_NODES];
  double cratio[SV_TREE_MAX_NODES];  // p(x) / q(x) at each child (inf: q(x) = 0 < p(x); nan: both 0)
  int wcnt[kTWaves];
  int nchild;
  Partial part[2][kTMaxNS];   // chunk partials of the position's target and draft rows
  double sub[kTMaxSub];       // sub-chunk masses of the current distribution
  double red[2 + kTWaves];
  double W;                   // their sum
  int pick, last;             // selection results
  int path[SV_TREE_MAX_NODES];  // the accepted nodes, in walk order
  int nchildp;                  // children of the prefetched position
  int wsA[2][kTMaxSub];         // per-wave row statistics (target, draft): M or arg-max,
  float wsB[2][kTMaxSub];       // and s or the maximum (statistics on demand)
};

// (M, s) of a stochastic row, or (max, lowest arg-max) of a greedy one, from
// K1's chunk partials (staged in LDS) merged in chunk order.
__device__ __forceinline__ void merged_row(const Partial *part, int NS, bool greedy, int &M, double &s, int &arg) {
  M = kEmptyM;
  s = 0.0;
  float mx = -INFINITY, v = -INFINITY;
  int ix = 0x7fffffff;
  for (int j = 0; j < NS; ++j) {
    const Partial q = part[j];
    if (greedy) merge_arg(v, ix, q.mx, q.mi);
    else merge_sm(M, s, mx, q.mi, q.s, q.mx);
  }
  arg = ix;
}

// Masses of w = max(0, e_p - r e_q) (or e_p without USEQ) over 2048-token
// sub-chunks of the position's rows, into sh.sub; their sum into sh.W.
template <int DT, bool USEQ>
__device__ __forceinline__ float tree_lane_mass(const u32x4 *tp, const u32x4 *dq, float c, float negMp, float negMq,
                                                float r) {
  constexpr int kN = kLaneElems / Elem<DT>::kVec;
  float acc = 0.0f;
#pragma unroll
  for (int u = 0; u < kN; ++u) {
    float zp[Elem<DT>::kVec], zq[Elem<DT>::kVec];
    widen_vec<DT>(tp[u], zp);
    if constexpr (USEQ) widen_vec<DT>(dq[u], zq);
#pragma unroll
    for (int e = 0; e < Elem<DT>::kVec; ++e) {
      const float ep = __builtin_amdgcn_exp2f(fmaf(zp[e], c, negMp));
      if constexpr (USEQ) acc += fmaxf(0.0f, fmaf(-__builtin_amdgcn_exp2f(fmaf(zq[e], c, negMq)), r, ep));
      else acc += ep;
    }
  }
  return acc;
}

// How the request's workgroups share a pass and meet after it.
struct TreeTeam {
  int w, NW;                 // this workgroup, workgroups per request
  unsigned long long *sub;   // [2][NSUB] per-request mass words (NW > 1), cleared before the walk
  unsigned long long *stat;  // [2][Wmax][4] per-request row-statistics words (statistics on demand)
  int Wmax;                  // waves a team can have (the words' stride)
  unsigned *err;             // set if a bounded wait ran out
  int pass;                  // exchanges done so far in this call
};

// A sub-chunk mass as the team exchanges it: pass number (from 1) in the high
// half, the mass rounded to fp32 in the low half, in one 64-bit word written
// and read with single device-scope atomic accesses, so that a reader that
// sees the pass number sees the mass.  The rounding moves a prefix of the
// masses by at most 6e-8 of their total.
__device__ __forceinline__ unsigned long long mass_word(int pass, double m) {
  return (static_cast<unsigned long long>(static_cast<unsigned>(pass)) << 32) |
         __float_as_uint(static_cast<float>(m));
}

// The sum of sh.sub[0, NSUB) into sh.W by wave 0 (a DPP tree per 64 entries,
// then the 64-entry totals in order): the same order in every workgroup.
__device__ __forceinline__ void tree_total(int NSUB, TreeShared &sh) {
  if (threadIdx.x < kWave) {
    const int lane = threadIdx.x;
    double W = 0.0;
    for (int j0 = 0; j0 < NSUB; j0 += kWave) W += wave_sum(j0 + lane < NSUB ? sh.sub[j0 + lane] : 0.0);
    if (lane == 0) sh.W = W;
  }
}

// A wave's registers of one 2048-token sub-chunk of a position's row pair
// (the interleaved layout of load_lane_fast), kept across the passes at that
// position when every wave of the request has at most one such sub-chunk.
template <int DT>
struct RowSlice {
  static constexpr int kN = kLaneElems / Elem<DT>::kVec;
  u32x4 t[kN], d[kN];
  bool valid;
};

// Wave gw of a team of `stride` waves takes sub-chunks gw, gw + stride, ...:
// first those wholly inside an aligned row (index < nfast), then the others (a
// partial last sub-chunk, or every sub-chunk of a row that is not aligned);
// this is its first index of the others.
__device__ __forceinline__ int first_guarded(int gw, int stride, int nfast) {
  return gw >= nfast ? gw : gw + (nfast - gw + stride - 1) / stride * stride;
}

template <int DT, bool USEQ>
__device__ __forceinline__ void tree_masses_of(const void *trow, const void *drow, bool aligned, int V, int NSUB, float c,
                               float negMp, float negMq, float r, const RowSlice<DT> &rs, TreeShared &sh,
                               TreeTeam &tm) {
  constexpr int kN = kLaneElems / Elem<DT>::kVec;
  const int lane = threadIdx.x & (kWave - 1), wave = threadIdx.x / kWave;
  // this wave's place among the request's NW x 4 waves
  const int gw = tm.w * kTWaves + wave, stride = tm.NW * kTWaves;
  unsigned long long *gsub = tm.NW > 1 ? tm.sub + (tm.pass & 1) * NSUB : nullptr;
  const int stamp = tm.pass + 1;
  auto put_mass = [&](int j, double v) {
    if (lane == 0) {
      if (gsub) put<true>(gsub + j, mass_word(stamp, v));
      else sh.sub[j] = v;
    }
  };
  // Sub-chunks wholly inside an aligned row: straight-line loads, the next one
  // requested while the current one is reduced (its index clamped to the last
  // such sub-chunk, so that the loads are unconditional and each wait covers
  // exactly the older sub-chunk).  A wave whose one sub-chunk is already in
  // registers (rs) reduces it directly.
  const int nfast = aligned ? min(NSUB, V / kSub) : 0;
  if (rs.valid) {  // uniform per wave: gw is the wave's only sub-chunk
    put_mass(gw, wave_sum(static_cast<double>(tree_lane_mass<DT, USEQ>(rs.t, rs.d, c, negMp, negMq, r))));
  } else if (gw < nfast) {
    u32x4 tp[kN], dq[kN], tn[kN], dn[kN];
    load_lane_fast<DT>(trow, static_cast<long>(gw) * kSub, lane, tp);
    if constexpr (USEQ) load_lane_fast<DT>(drow, static_cast<long>(gw) * kSub, lane, dq);
    for (int j = gw; j < nfast; j += stride) {
      const long jn = min(j + stride, nfast - 1);
      load_lane_fast<DT>(trow, jn * kSub, lane, tn);
      if constexpr (USEQ) load_lane_fast<DT>(drow, jn * kSub, lane, dn);
      put_mass(j, wave_sum(static_cast<double>(tree_lane_mass<DT, USEQ>(tp, dq, c, negMp, negMq, r))));
#pragma unroll
      for (int u = 0; u < kN; ++u) {
        tp[u] = tn[u];
        if constexpr (USEQ) dq[u] = dn[u];
      }
    }
  }
  // the rest: guarded loads, one sub-chunk at a time
  for (int j = rs.valid ? NSUB : first_guarded(gw, stride, nfast); j < NSUB; j += stride) {
    u32x4 tp[kN], dq[kN];
    load_lane_raw<DT>(trow, aligned, static_cast<long>(j) * kSub, lane, V, tp);
    if constexpr (USEQ) load_lane_raw<DT>(drow, aligned, static_cast<long>(j) * kSub, lane, V, dq);
    put_mass(j, wave_sum(static_cast<double>(tree_lane_mass<DT, USEQ>(tp, dq, c, negMp, negMq, r))));
  }
  if (gsub) {
    // wave 0 polls the request's words until each carries this pass's number
    // (bounded: if one never arrives the error word is set), the other waves
    // wait at the barrier.  The two copies alternate between passes: a
    // workgroup writes copy p + 1 only after reading all of copy p - 1's
    // successor p, so a copy is never overwritten while a reader waits on it.
    if (threadIdx.x < kWave) {
      for (int j0 = 0; j0 < NSUB; j0 += kWave) {
        const int j = j0 + lane;
        unsigned long long word = 0;
        for (unsigned it = 0;; ++it) {
          if (j < NSUB) word = get<true>(gsub + j);
          const bool ready = j >= NSUB || static_cast<int>(word >> 32) == stamp;
          if (__all(ready)) break;
          if (it >= kSpinLimit) {
            if (lane == 0) put<true>(tm.err, 1u);
            break;
          }
          __builtin_amdgcn_s_sleep(1);
        }
        if (j < NSUB) sh.sub[j] = static_cast<double>(__uint_as_float(static_cast<unsigned>(word)));
      }
    }
    ++tm.pass;
  }
  tree_barrier();
  tree_total(NSUB, sh);
  tree_barrier();
}

template <int DT>
__device__ __forceinline__ void tree_masses(const void *trow, const void *drow, bool aligned, int V, int NSUB, float c,
                            float negMp, float negMq, float r, bool use_q, const RowSlice<DT> &rs, TreeShared &sh,
                            TreeTeam &tm) {
  if (use_q) tree_masses_of<DT, true>(trow, drow, aligned, V, NSUB, c, negMp, negMq, r, rs, sh, tm);
  else tree_masses_of<DT, false>(trow, drow, aligned, V, NSUB, c, negMp, negMq, r, rs, sh, tm);
}

// Inverse CDF over the masses in sh.sub (of the same w as tree_masses): the
// lowest token with mass whose running prefix exceeds u * W; if rounding
// leaves none, the last token with mass.
// The sub-chunk of the draw (sh.pick), the mass before it (sh.red[0]) and the
// target u W (sh.red[1]), by wave 0 from sh.sub / sh.W; every thread calls.
__device__ __forceinline__ void tree_crossing(int NSUB, float u, TreeShared &sh) {
  const int tid = threadIdx.x, lane = tid & (kWave - 1);
  if (tid < kWave) {  // wave 0: the lowest sub-chunk with mass whose inclusive prefix exceeds u W
    const double target = static_cast<double>(u) * sh.W;
    double run = 0.0, base = 0.0, base_last = 0.0;
    int sub = -1, lastm = -1;
    for (int j0 = 0; j0 < NSUB && sub < 0; j0 += kWave) {
      const int j = j0 + lane;
      const double m = j < NSUB ? sh.sub[j] : 0.0;
      const double incl = wave_scan(m, lane);
      const unsigned long long hit = __ballot(j < NSUB && m > 0.0 && target < run + incl);
      const unsigned long long has = __ballot(j < NSUB && m > 0.0);
      if (hit) {
        const int L = __ffsll(static_cast<long long>(hit)) - 1;
        sub = j0 + L;
        base = run + lane_value(incl - m, L);
      } else if (has) {
        const int L = 63 - __clzll(static_cast<long long>(has));
        lastm = j0 + L;
        base_last = run + lane_value(incl - m, L);
      }
      run += lane_value(incl, kWave - 1);
    }
    if (sub < 0) {  // rounding left u W at the very end: the last sub-chunk with mass
      sub = lastm >= 0 ? lastm : 0;
      base = lastm >= 0 ? base_last : 0.0;
    }
    if (lane == 0) {
      sh.pick = sub;
      sh.red[0] = base;
      sh.red[1] = target;
    }
  }
  tree_barrier();
}

// The token of the draw, read again from memory by one workgroup (the
// crossing from tree_crossing): four contiguous tokens per thread.
template <int DT>
__device__ __forceinline__ int tree_select(const void *trow, const void *drow, int V, float c, float negMp,
                                           float negMq, float r, bool use_q, TreeShared &sh) {
  const int tid = threadIdx.x, lane = tid & (kWave - 1), wave = tid / kWave;
  const int sub = sh.pick;
  const double base = sh.red[0], target = sh.red[1];
  tree_barrier();
  // four contiguous tokens per thread, in token order through waves and lanes
  constexpr int kPer = kSub / kTBlock;
  const long first = static_cast<long>(sub) * kSub + static_cast<long>(tid) * kPer;
  float w[kPer];
  double lsum = 0.0;
#pragma unroll
  for (int e = 0; e < kPer; ++e) {
    const long t = first + e;
    if (t < V) {
      const float ep = __builtin_amdgcn_exp2f(fmaf(load_one<DT>(trow, t), c, negMp));
      w[e] = use_q ? fmaxf(0.0f, fmaf(-__builtin_amdgcn_exp2f(fmaf(load_one<DT>(drow, t), c, negMq)), r, ep)) : ep;
    } else {
      w[e] = 0.0f;
    }
    lsum += static_cast<double>(w[e]);
  }
  const double incl = wave_scan(lsum, lane);
  if (lane == kWave - 1) sh.red[2 + wave] = incl;  // red[2 .. 2 + kTWaves) is free after the broadcast
  tree_barrier();
  double before = base;
  for (int q = 0; q < wave; ++q) before += sh.red[2 + q];
  if (tid == 0) {
    sh.pick = 0x7fffffff;
    sh.last = -1;
  }
  tree_barrier();
  double acc = before + (incl - lsum);
  int cand = -1, lastp = -1;
#pragma unroll
  for (int e = 0; e < kPer; ++e) {
    if (w[e] > 0.0f) {
      lastp = static_cast<int>(first + e);
      acc += static_cast<double>(w[e]);
      if (cand < 0 && target < acc) cand = static_cast<int>(first + e);
    }
  }
  if (cand >= 0) atomicMin(&sh.pick, cand);
  if (lastp >= 0) atomicMax(&sh.last, lastp);
  tree_barrier();
  int tok = sh.pick;
  if (tok == 0x7fffffff) tok = sh.last >= 0 ? sh.last : static_cast<int>(static_cast<long>(sub) * kSub);
  tree_barrier();
  return tok;
}

// A lane's tokens of one sub-chunk (interleaved layout, base = its first
// token): the largest value and its lowest index folded into (v, i); the first
// token is taken even when it is -inf, so an all -inf row yields index 0.
template <int DT>
__device__ __forceinline__ void lane_argmax(const u32x4 *raw, long base, int lane, float &v, int &i) {
  constexpr int kV = Elem<DT>::kVec;
#pragma unroll
  for (int u = 0; u < kLaneElems / kV; ++u) {
    float x[kV];
    widen_vec<DT>(raw[u], x);
#pragma unroll
    for (int e = 0; e < kV; ++e) {
      const int idx = static_cast<int>(base + static_cast<long>(u * kWave + lane) * kV + e);
      if (x[e] > v || i == INT_MAX) {
        v = x[e];
        i = idx;
      }
    }
  }
}

// A team-exchanged statistic: the exchange number in the high half, 32 bits of
// payload (an int, or a float's bits) in the low half.
__device__ __forceinline__ unsigned long long stat_word(int stamp, unsigned bits) {
  return (static_cast<unsigned long long>(static_cast<unsigned>(stamp)) << 32) | bits;
}

// The statistics of a position's rows, computed by the team (no K1): each wave
// folds its sub-chunks of the target row (and of the draft row when need_q) as
// K1 folds a tile, its lanes merge with DPP (the largest M, each sum rescaled to
// it by an exact power of two, one fp64 sum; greedy: the maximum, then the
// lowest index holding it), and the waves' results go to every workgroup of
// the team (tagged words, or LDS when the team is one workgroup), which merges
// them in wave order: (M, s) into sh.wsA/wsB, then the caller's merge.  The
// sub-chunks are shared out as in tree_masses_of; the wave's one fast
// sub-chunk is taken from its registers (rs) when it has them.
template <int DT>
__device__ __forceinline__ int tree_stats(const void *trow, const void *drow, bool al, int V, int NSUB, float c,
                                          bool greedy, bool need_q, const RowSlice<DT> &rs, TreeShared &sh,
                                          TreeTeam &tm) {
  constexpr int kN = kLaneElems / Elem<DT>::kVec;
  const int lane = threadIdx.x & (kWave - 1), wave = threadIdx.x / kWave;
  const int gw = tm.w * kTWaves + wave, stride = tm.NW * kTWaves;
  const int nfast = al ? min(NSUB, V / kSub) : 0;
  const int nwv = min(stride, NSUB);  // waves that hold a sub-chunk
  int Mt = kEmptyM, Mq = kEmptyM;
  double st = 0.0, sq = 0.0;
  float mt = -INFINITY, mq = -INFINITY;
  float gv = -INFINITY;
  int gi = INT_MAX;
  auto fold = [&](const u32x4 *tv, const u32x4 *dv, long base) {
    if (greedy) {
      lane_argmax<DT>(tv, base, lane, gv, gi);
    } else {
      fold_tile<DT, kN>(tv, c, Mt, st, mt);
      if (need_q) fold_tile<DT, kN>(dv, c, Mq, sq, mq);
    }
  };
  if (rs.valid) {  // uniform per wave: gw is the wave's only sub-chunk
    fold(rs.t, rs.d, static_cast<long>(gw) * kSub);
  } else {
    for (int j = gw; j < nfast; j += stride) {
      u32x4 tv[kN], dv[kN];
      load_lane_fast<DT>(trow, static_cast<long>(j) * kSub, lane, tv);
      if (need_q) load_lane_fast<DT>(drow, static_cast<long>(j) * kSub, lane, dv);
      fold(tv, dv, static_cast<long>(j) * kSub);
    }
  }
  for (int j = rs.valid ? NSUB : first_guarded(gw, stride, nfast); j < NSUB; j += stride) {
    u32x4 tv[kN], dv[kN];
    load_lane_raw<DT>(trow, al, static_cast<long>(j) * kSub, lane, V, tv);
    if (need_q) load_lane_raw<DT>(drow, al, static_cast<long>(j) * kSub, lane, V, dv);
    fold(tv, dv, static_cast<long>(j) * kSub);
  }
  // the wave's results: (A, B) = (M, s) or (arg-max, max) per row
  int A0, A1 = kEmptyM;
  float B0, B1 = 0.0f;
  if (greedy) {
    const float vm = wave_max_f32(gv);
    A0 = wave_ext_i32<false>(gv == vm ? gi : INT_MAX);
    B0 = vm;
  } else {
    A0 = wave_ext_i32<true>(Mt);
    B0 = static_cast<float>(wave_sum(ldexp(st, Mt - A0)));
    if (need_q) {
      A1 = wave_ext_i32<true>(Mq);
      B1 = static_cast<float>(wave_sum(ldexp(sq, Mq - A1)));
    }
  }
  const int nk = need_q ? 4 : 2;  // words per wave
  if (tm.NW > 1) {
    unsigned long long *wd = tm.stat + static_cast<long>(tm.pass & 1) * tm.Wmax * 4;
    const int stamp = tm.pass + 1;
    if (lane == 0 && gw < nwv) {
      put<true>(wd + gw * 4 + 0, stat_word(stamp, static_cast<unsigned>(A0)));
      put<true>(wd + gw * 4 + 1, stat_word(stamp, __float_as_uint(B0)));
      if (need_q) {
        put<true>(wd + gw * 4 + 2, stat_word(stamp, static_cast<unsigned>(A1)));
        put<true>(wd + gw * 4 + 3, stat_word(stamp, __float_as_uint(B1)));
      }
    }
    // wave 0 polls the team's words until each carries this exchange's number
    // (bounded: if one never arrives the error word is set); the two copies
    // alternate between exchanges as the mass words do
    if (wave == 0) {  // lane l polls the words of waves l, l + 64, ..., all of a wave's words at once
      for (int w0 = 0; w0 < nwv; w0 += kWave) {
        const int w = w0 + lane;
        const bool mine = w < nwv;
        unsigned long long word[4] = {0ull, 0ull, 0ull, 0ull};
        for (unsigned it = 0;; ++it) {
          bool ready = true;
#pragma unroll
          for (int k = 0; k < 4; ++k) {
            if (mine && k < nk) word[k] = get<true>(wd + w * 4 + k);
            ready = ready && (!mine || k >= nk || static_cast<int>(word[k] >> 32) == stamp);
          }
          if (__all(ready)) break;
          if (it >= kSpinLimit) {
            if (lane == 0) put<true>(tm.err, 1u);
            break;
          }
          __builtin_amdgcn_s_sleep(1);
        }
        if (mine) {
          sh.wsA[0][w] = static_cast<int>(static_cast<unsigned>(word[0]));
          sh.wsB[0][w] = __uint_as_float(static_cast<unsigned>(word[1]));
          sh.wsA[1][w] = static_cast<int>(static_cast<unsigned>(word[2]));
          sh.wsB[1][w] = __uint_as_float(static_cast<unsigned>(word[3]));
        }
      }
    }
    ++tm.pass;
  } else if (lane == 0 && gw < nwv) {
    sh.wsA[0][gw] = A0;
    sh.wsB[0][gw] = B0;
    sh.wsA[1][gw] = A1;
    sh.wsB[1][gw] = B1;
  }
  tree_barrier();
  return nwv;
}

// The merged statistics of row t (0: target, 1: draft) from the per-wave
// results in sh.wsA/wsB, by one wave (every lane calls; lane l takes waves l,
// l + 64, ...): the same DPP merge as within a wave, 64 waves at a time.
__device__ __forceinline__ void merged_waves(const TreeShared &sh, int t, int nwv, bool greedy, int lane, int &M,
                                             double &s, int &arg) {
  M = kEmptyM;
  s = 0.0;
  float mx = -INFINITY, v = -INFINITY;
  int ix = INT_MAX;
  for (int w0 = 0; w0 < nwv; w0 += kWave) {
    const int w = w0 + lane;
    const bool in = w < nwv;
    if (greedy) {
      const float b = in ? sh.wsB[t][w] : -INFINITY;
      const float vm = wave_max_f32(b);
      merge_arg(v, ix, vm, wave_ext_i32<false>(in && b == vm ? sh.wsA[t][w] : INT_MAX));
    } else {
      const int a = in ? sh.wsA[t][w] : kEmptyM;
      const int Mw = wave_ext_i32<true>(a);
      const double sw = wave_sum(in ? ldexp(static_cast<double>(sh.wsB[t][w]), a - Mw) : 0.0);
      merge_sm(M, s, mx, Mw, sw, 0.0f);
    }
  }
  arg = ix;
}

// Zeroes the walk's exchange words before a walk with statistics on demand.
__global__ __launch_bounds__(kBlock) void k_tree_clear(unsigned long long *__restrict__ words, long n) {
  for (long i = static_cast<long>(blockIdx.x) * kBlock + threadIdx.x; i < n; i += static_cast<long>(gridDim.x) * kBlock)
    words[i] = 0ull;
}

template <int DT, bool OD>
__global__ __launch_bounds__(kTBlock) void k_tree_walk(
    const void *__restrict__ target, const void *__restrict__ draft, const int32_t *__restrict__ parent,
    const int32_t *__restrict__ tokens, const int32_t *__restrict__ num_nodes, const float *__restrict__ u_accept,
    const float *__restrict__ u_sample, const float *__restrict__ temps, int Nmax, int V, int NS,
    const Partial *__restrict__ part, int32_t *__restrict__ count, int32_t *__restrict__ out_tokens,
    int32_t *__restrict__ out_nodes, int NW, unsigned long long *__restrict__ tsub, unsigned *__restrict__ terr,
    const void *__restrict__ spare, unsigned long long *__restrict__ tstat, int Wmax) {
  const int b = blockIdx.x / NW, tid = threadIdx.x;
  const int rows = 2 * Nmax + 1;
  const int N = request_len(num_nodes, Nmax, b);
  const float T = temps[b];
  const float us = u_sample[b];
  const bool greedy = !(T > 0.0f);
  const float c = greedy ? 0.0f : temp_scale(T);
  const int NSUB = (V + kSub - 1) / kSub;
  TreeTeam tm;
  tm.w = blockIdx.x - b * NW;
  // a greedy walk with K1's statistics makes no pass: workgroup 0 alone
  tm.NW = (greedy && !OD) ? 1 : NW;
  tm.sub = tsub + static_cast<long>(b) * 2 * NSUB;  // cleared before the walk
  tm.stat = OD ? tstat + static_cast<long>(b) * 2 * Wmax * 4 : nullptr;
  tm.Wmax = Wmax;
  tm.err = terr;
  tm.pass = 0;
  if (tm.w >= tm.NW) return;  // uniform per workgroup
  const bool lead = tm.w == 0;     // writes the outputs
  __shared__ TreeShared sh;
  __shared__ int s_hit, s_arg, s_Mp, s_Mq;
  __shared__ double s_sp, s_sq;
  for (int n = tid; n < Nmax; n += kTBlock) {
    int pa = -2, x = -1;
    if (n < N) {
      pa = parent[static_cast<long>(b) * Nmax + n];
      x = tokens[static_cast<long>(b) * Nmax + n];
      if (pa < -1 || pa >= n) pa = -2;  // not a valid child of anything
    }
    sh.parent[n] = pa;
    sh.token[n] = x;
  }
  tree_barrier();
  const size_t eb = Elem<DT>::kBytes;
  const int lane = tid & (kWave - 1), wave = tid / kWave;
  auto target_row = [&](int p) -> const void * {
    return static_cast<const char *>(target) + (static_cast<long>(b) * (Nmax + 1) + p) * V * eb;
  };
  auto draft_row = [&](int p) -> const void * {  // position Nmax has no child, so no draft row
    return p < Nmax ? static_cast<const char *>(draft) + (static_cast<long>(b) * Nmax + p) * V * eb : nullptr;
  };
  // position p's children in node order, into list (a block-wide compaction)
  auto children = [&](int p, int *list) -> int {
    const bool is_child = tid < N && tid >= p && sh.parent[tid] == p - 1;
    const unsigned long long mask = __ballot(is_child);
    if (lane == 0) sh.wcnt[wave] = __popcll(mask);
    tree_barrier();
    int n = 0, before = 0;
    for (int w = 0; w < kTWaves; ++w) {
      if (w < wave) before += sh.wcnt[w];
      n += sh.wcnt[w];
    }
    if (is_child) list[before + __popcll(mask & ((1ull << lane) - 1ull))] = tid;
    tree_barrier();
    return n;
  };
  // each child's two logits and its uniform, as raw bits (the threads past the
  // first two waves, a thread per child and, past their count, a second)
  constexpr int kGather = kTBlock - 2 * kWave;  // threads that gather children
  static_assert(2 * kGather >= SV_TREE_MAX_NODES, "at most two children per gathering thread");
  const int jc = tid - 2 * kWave;
  auto gather = [&](const int *list, int n, const void *tr, const void *dr, unsigned (&z)[2][3]) {
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const int j = jc + h * kGather;
      z[h][0] = z[h][1] = 0u;
      z[h][2] = __float_as_uint(2.0f);  // 2 rejects
      if (!greedy && jc >= 0 && j < n) {
        const int nd = list[j], x = sh.token[nd];
        if (x >= 0 && x < V) {  // an id outside the vocabulary is rejected, never dereferenced
          z[h][0] = load_bits<DT>(tr, x);
          z[h][1] = load_bits<DT>(dr, x);
          z[h][2] = __float_as_uint(u_accept[static_cast<long>(b) * Nmax + nd]);
        }
      }
    }
  };
  // the wave's sub-chunk of a position's row pair, kept in registers for the
  // passes at that position when each wave has at most one (bf16 only: an fp32
  // slice is twice the registers)
  auto load_slice = [&](const void *tr, const void *dr, bool al, RowSlice<DT> &r) {
    const int gw = tm.w * kTWaves + wave, stride = tm.NW * kTWaves;
    r.valid = DT == SV_BF16 && (OD || (!greedy && dr != nullptr)) && gw < NSUB && gw + stride >= NSUB;
    if constexpr (DT == SV_BF16) {
      const bool need_d = dr && !greedy;
      if (r.valid && !(al && static_cast<long>(gw + 1) * kSub <= V)) {  // a guarded sub-chunk (uniform per wave)
        load_lane_raw<DT>(tr, al, static_cast<long>(gw) * kSub, lane, V, r.t);
        if (need_d) load_lane_raw<DT>(dr, al, static_cast<long>(gw) * kSub, lane, V, r.d);
        else load_lane_fast<DT>(spare, 0, lane, r.d);
      } else {
        // unconditional loads (from the workspace's spare block when the wave
        // holds no slice), so that waiting for the loads before them never
        // waits for these
        const void *ts = r.valid ? tr : spare, *ds = r.valid && need_d ? dr : spare;
        const long off = r.valid ? static_cast<long>(gw) * kSub : 0;
        load_lane_fast<DT>(ts, off, lane, r.t);
        load_lane_fast<DT>(ds, off, lane, r.d);
      }
    }
  };
  // With statistics on demand, the position of the current one's first child
  // (the most likely next) is prefetched while this one is decided: its
  // children, their logits and the row slices.
  // (the children's list, logits and uniforms by the last wave alone, which
  // holds child j's in lane j % 64, slot j / 64; no workgroup barrier)
  int ppos = -1;
  unsigned zc_pf[kTMaxNodesPerLane][3];
  RowSlice<DT> rs_pf;
  int pos = 0, depth = 0;
  for (;;) {
    const void *trow = target_row(pos);
    const void *drow = draft_row(pos);
    const bool al = ((reinterpret_cast<uintptr_t>(trow) | reinterpret_cast<uintptr_t>(drow)) & 15u) == 0;
    // everything the position needs, requested together (one round trip): with
    // K1, the chunk partials of its two rows (wave 0: the target row, wave 1:
    // the draft row; lane j: chunks j and j + 64); each child's two logits and
    // its uniform; every wave's sub-chunk of the row pair.  A prefetched
    // position has them already.
    const bool pre = OD && pos == ppos;  // uniform across the team
    const bool want_part = !OD && (wave == 0 || (wave == 1 && !greedy && pos < N));
    int nchild;
    unsigned zc[2][3];
    RowSlice<DT> rs;
    if (pre) {
      nchild = sh.nchildp;
      for (int j = tid; j < nchild; j += kTBlock) sh.child[j] = sh.childp[j];
      if (wave == kTWaves - 1 && !greedy) {
#pragma unroll
        for (int h = 0; h < kTMaxNodesPerLane; ++h) {
          const int j = lane + h * kWave;
          if (j < nchild) {
            sh.czp[j] = bits_value<DT>(zc_pf[h][0]);
            sh.czq[j] = bits_value<DT>(zc_pf[h][1]);
            sh.cu[j] = __uint_as_float(zc_pf[h][2]);
          }
        }
      }
      rs = rs_pf;
    } else {
      nchild = children(pos, sh.child);
      u32x4 pv0 = {0u, 0u, 0u, 0u}, pv1 = {0u, 0u, 0u, 0u};  // the records as raw 16-byte vectors
      if (want_part) {
        const u32x4 *src = reinterpret_cast<const u32x4 *>(part) +
                           (static_cast<long>(b) * rows + (wave == 0 ? pos : Nmax + 1 + pos)) * NS;
        if (lane < NS) pv0 = src[lane];
        if (lane + kWave < NS) pv1 = src[lane + kWave];
      }
      gather(sh.child, nchild, trow, drow, zc);
      load_slice(trow, drow, al, rs);
      if (want_part) {
        u32x4 *dst = reinterpret_cast<u32x4 *>(sh.part[wave]);
        if (lane < NS) dst[lane] = pv0;
        if (lane + kWave < NS) dst[lane + kWave] = pv1;
      }
    }
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const int j = jc + h * kGather;
      if (!pre && !greedy && jc >= 0 && j < nchild) {
        sh.czp[j] = bits_value<DT>(zc[h][0]);
        sh.czq[j] = bits_value<DT>(zc[h][1]);
        sh.cu[j] = __uint_as_float(zc[h][2]);
      }
    }
    tree_barrier();
    // the two rows' statistics (target by thread 0, draft by the first lane of
    // wave 1), from K1's chunk partials or computed here by the team
    if constexpr (OD) {
      const bool need_q = !greedy && nchild > 0;
      const int nwv = tree_stats<DT>(trow, drow, al, V, NSUB, c, greedy, need_q, rs, sh, tm);
      if (wave == 0) {
        int M, arg;
        double s;
        merged_waves(sh, 0, nwv, greedy, lane, M, s, arg);
        if (lane == 0) {
          s_Mp = M;
          s_sp = s;
          s_arg = arg;
        }
      }
      if (wave == 1 && need_q) {
        int M, arg;
        double s;
        merged_waves(sh, 1, nwv, false, lane, M, s, arg);
        if (lane == 0) {
          s_Mq = M;
          s_sq = s;
        }
      }
    } else {
      if (tid == 0) {
        int M, arg;
        double s;
        merged_row(sh.part[0], NS, greedy, M, s, arg);
        s_Mp = M;
        s_sp = s;
        s_arg = arg;
      }
      if (tid == kWave && !greedy && pos < N) {
        int arg;
        merged_row(sh.part[1], NS, false, s_Mq, s_sq, arg);
      }
    }
    tree_barrier();
    if constexpr (OD) {
      // the prefetch of the likely next position: the first child's (for a
      // greedy walk, the child equal to the arg-max: the next one for sure)
      int nxt = -1;
      if (greedy) {
        for (int j = 0; j < nchild && nxt < 0; ++j)
          if (sh.token[sh.child[j]] == s_arg) nxt = sh.child[j];
      } else {
        nxt = nchild > 0 ? sh.child[0] : -1;
      }
      ppos = nxt >= 0 ? nxt + 1 : -1;
      if (ppos >= 0) {  // uniform across the team
        const void *tp = target_row(ppos), *dp = draft_row(ppos);
        const bool alp = ((reinterpret_cast<uintptr_t>(tp) | reinterpret_cast<uintptr_t>(dp)) & 15u) == 0;
        load_slice(tp, dp, alp, rs_pf);
        if (wave == kTWaves - 1) {
          // children of ppos are nodes >= ppos: a wave-level compaction, 64 at a time
          int n = 0;
          for (int base = ppos; base < N; base += kWave) {
            const int t = base + lane;
            const bool is_child = t < N && sh.parent[t] == ppos - 1;
            const unsigned long long m = __ballot(is_child);
            if (is_child) sh.childp[n + __popcll(m & ((1ull << lane) - 1ull))] = t;
            n += __popcll(m);
          }
          if (lane == 0) sh.nchildp = n;
          __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront", "local");
          __builtin_amdgcn_wave_barrier();
          __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront", "local");
#pragma unroll
          for (int h = 0; h < kTMaxNodesPerLane; ++h) {
            const int j = lane + h * kWave;
            zc_pf[h][0] = zc_pf[h][1] = 0u;
            zc_pf[h][2] = __float_as_uint(2.0f);  // 2 rejects
            if (!greedy && j < n) {
              const int nd = sh.childp[j], x = sh.token[nd];
              if (x >= 0 && x < V) {  // an id outside the vocabulary is rejected, never dereferenced
                zc_pf[h][0] = load_bits<DT>(tp, x);
                zc_pf[h][1] = load_bits<DT>(dp, x);
                zc_pf[h][2] = __float_as_uint(u_accept[static_cast<long>(b) * Nmax + nd]);
              }
            }
          }
        }
      }
    }
    // every child's p(x)/q(x) at once, one exponential each:
    // 2^((zp - zq) c - (Mp - Mq)) * s'_q / s'_p (the logit difference is exact)
    for (int j = tid; !greedy && j < nchild; j += kTBlock) {
      const double d = (static_cast<double>(sh.czp[j]) - static_cast<double>(sh.czq[j])) * static_cast<double>(c) -
                       static_cast<double>(s_Mp - s_Mq);
      sh.cratio[j] = exp2(d) * (s_sq / s_sp);
    }
    tree_barrier();
    int hit = -1;
    if (greedy) {
      if (tid == 0) {
        for (int j = 0; j < nchild && hit < 0; ++j)
          if (sh.token[sh.child[j]] == s_arg) hit = sh.child[j];
        s_hit = hit;
      }
      tree_barrier();
      hit = s_hit;
      if (hit < 0) {
        if (lead && tid == 0) out_tokens[static_cast<long>(b) * (Nmax + 1) + depth] = s_arg;
        break;
      }
    } else {
      const int Mp = s_Mp;
      const double sp = s_sp;
      const float negMp = -static_cast<float>(Mp);
      const int Mq = nchild > 0 ? s_Mq : 0;
      const double sq = nchild > 0 ? s_sq : 1.0;
      double cc = 0.0, Z = 1.0;  // current target: max(0, p - cc q) / Z
      bool masses_current = false;
      for (int j = 0; j < nchild; ++j) {
        if (tid == 0) {
          // the current target over q at x: max(0, p - cc q) / (Z q) = max(0, p/q - cc) / Z
          const double ratio = sh.cratio[j];
          const double a = fmin(1.0, fmax(0.0, ratio - cc) / Z);
          s_hit = static_cast<double>(sh.cu[j]) < a ? sh.child[j] : -1;
        }
        tree_barrier();
        hit = s_hit;
        tree_barrier();
        if (hit >= 0) break;
        // rejected: the next target is max(0, p - (cc + Z) q) / Z'
        cc += Z;
        const float r = static_cast<float>(cc * sp / sq);
        tree_masses<DT>(trow, drow, al, V, NSUB, c, negMp, -static_cast<float>(Mq), r, true, rs, sh, tm);
        const double W = sh.W;
        if (W > 0.0) {
          Z = W / sp;
          masses_current = true;
        } else {  // zero residual mass: back to the position's p
          cc = 0.0;
          Z = 1.0;
          masses_current = false;
        }
      }
      if (hit < 0) {
        // every child rejected, or none: draw from the current target
        const bool use_q = cc > 0.0;
        const float r = use_q ? static_cast<float>(cc * sp / sq) : 0.0f;
        if (!masses_current) {
          if (OD && !use_q && tm.NW * kTWaves >= NSUB) {
            // p's sub-chunk masses are the waves' statistics already exchanged
            // (one sub-chunk per wave), rescaled to the row's M: no pass
            for (int j = tid; j < NSUB; j += kTBlock)
              sh.sub[j] = ldexp(static_cast<double>(sh.wsB[0][j]), sh.wsA[0][j] - Mp);
            tree_barrier();
            tree_total(NSUB, sh);
            tree_barrier();
          } else {
            tree_masses<DT>(trow, drow, al, V, NSUB, c, negMp, -static_cast<float>(Mq), r, use_q, rs, sh, tm);
          }
        }
        // every workgroup finds the crossing from the same masses; the wave that
        // holds that sub-chunk in registers draws from them, else the lead
        // workgroup reads it again
        tree_crossing(NSUB, us, sh);
        const int sub = sh.pick;
        const int stride = tm.NW * kTWaves;
        // (wave `sub` of the team, if there is one, holds it when that is its
        // only sub-chunk: rs.valid there)
        const bool held = DT == SV_BF16 && (OD || drow != nullptr) && sub < stride && sub + stride >= NSUB;
        int32_t *dst = out_tokens + static_cast<long>(b) * (Nmax + 1) + depth;
        if (held) {
          if (tm.w * kTWaves + wave == sub) {  // uniform per wave: this wave's rs holds the sub-chunk
            SelParams sp;
            sp.mode = use_q ? 1 : 2;
            sp.k = depth;
            sp.c = c;
            sp.negMp = negMp;
            sp.negMq = -static_cast<float>(Mq);
            sp.r = r;
            sp.ip = 0.0;
            sp.tau_p = sp.tau_q = -INFINITY;
            draw_held<DT, false>(rs.t, rs.d, sp, false, static_cast<long>(sub) * kSub, sh.red[0], sh.red[1], lane,
                                 dst);
          }
        } else if (lead) {  // uniform per workgroup
          const int tok = tree_select<DT>(trow, drow, V, c, negMp, -static_cast<float>(Mq), r, use_q, sh);
          if (tid == 0) *dst = tok;
        }
        break;
      }
    }
    // accepted node `hit`: the path is kept in LDS (written out after the walk)
    if (lead && tid == 0) sh.path[depth] = hit;
    ++depth;
    pos = hit + 1;
    // Every load of this position has long arrived (a row slice no pass used,
    // at the latest); waiting for them here lets the next position's waits
    // count only its own loads.
    __builtin_amdgcn_s_waitcnt(kWaitVmcnt0);
    tree_barrier();
  }
  // the accepted path, then the padding after the last token and node, written
  // last: the token at `depth` may come from another workgroup of the team, and
  // a store of this workgroup to the same word could reach memory after it
  if (lead) {
    for (int t = tid; t < depth; t += kTBlock) {
      const int n = sh.path[t];
      out_tokens[static_cast<long>(b) * (Nmax + 1) + t] = sh.token[n];
      out_nodes[static_cast<long>(b) * Nmax + t] = n;
    }
    for (int t = depth + 1 + tid; t <= Nmax; t += kTBlock) out_tokens[static_cast<long>(b) * (Nmax + 1) + t] = -1;
    for (int t = depth + tid; t < Nmax; t += kTBlock) out_nodes[static_cast<long>(b) * Nmax + t] = -1;
    if (tid == 0) count[b] = depth;
  }
}

// ================================================================== small problems
// The same step as K1 + K2 (temperature softmax, acceptance test and first
// rejection, residual or bonus draw; the pages' sections cited at the top of
// this file) for a request whose rows hold at most kSmElems logits in all
// ((2 gamma + 1) V): one workgroup, one kernel.  Its rows are read once into LDS
// (one batch of loads), and the statistics, the decision and the draw follow
// on chip, with no hand-over between workgroups and no second launch.  For
// such rows the two-kernel path is a chain of launches and round trips over a
// few kilobytes.
//   stage     every needed logit of the request -> LDS (fp32), rows in order;
//   stats     wave w takes rows w, w + kSmWaves, ...: (M, s) as K1 computes
//             them (integer M of the lane's maximum, exact power-of-two
//             merges), or the maximum and its lowest index for a greedy row;
//   decide    wave 0, as decide_request: fp64 ratio from the staged logits at
//             the draft tokens, ballot for the first rejection;
//   draw      thread t takes the contiguous tokens [t C, (t+1) C) of the row
//             sampled (C = ceil(V / kSmBlock)); a block scan of the threads'
//             fp64 sums gives every thread its prefix, and the thread whose
//             range holds u*Z walks its tokens.
constexpr int kSmBlock = 1024;
constexpr int kSmWaves = kSmBlock / kWave;
constexpr int kSmElems = 12288;                  // logits staged in LDS (48 KB)
constexpr int kSmBatch = kSmElems / kSmBlock;    // loads in flight per thread
constexpr int kSmRun = 16;                       // staged logits a lane folds at a time

struct SmallArgs {
  const void *target, *draft;
  const int32_t *tokens;
  const float *u_accept, *u_sample, *temps;
  float scalar_T;
  const int32_t *lens;
  int gamma, V;
  int32_t *count, *out;
  sv_debug dbg;
};

template <int DT, int KIND>
__global__ __launch_bounds__(kSmBlock) void k_small_verify(SmallArgs a) {
  extern __shared__ float zs[];  // [2 gamma + 1][V] staged logits, target rows first
  __shared__ int sh_M[2 * SV_GAMMA_MAX + 1], sh_arg[2 * SV_GAMMA_MAX + 1];
  __shared__ double sh_s[2 * SV_GAMMA_MAX + 1];
  __shared__ float sh_mx[2 * SV_GAMMA_MAX + 1];
  __shared__ double sh_wtot[kSmWaves];
  __shared__ int sh_k;
  const int b = blockIdx.x;
  const int tid = threadIdx.x, lane = tid & (kWave - 1), wave = tid / kWave;
  const int gamma = a.gamma, V = a.V, rows = 2 * gamma + 1;
  // one round trip for everything a uniform batch needs: the request's target
  // rows (contiguous), its draft rows, its draft tokens and uniforms.  With
  // per-request temperatures the draft rows and uniforms wait for T (a greedy
  // request reads neither); padding rows past a ragged request's length are
  // staged but never used.
  const int nt = (gamma + 1) * V, nd = gamma * V;
  const char *tb = static_cast<const char *>(a.target) + static_cast<long>(b) * nt * Elem<DT>::kBytes;
  const char *db =  // NULL for a batch that reads no draft row
      a.draft ? static_cast<const char *>(a.draft) + static_cast<long>(b) * nd * Elem<DT>::kBytes : nullptr;
  float bt[kSmBatch], bd[kSmBatch];
#pragma unroll
  for (int q = 0; q < kSmBatch; ++q) {
    const int e = q * kSmBlock + tid;
    bt[q] = e < nt ? load_one<DT>(tb, e) : -INFINITY;
  }
  const int x = (wave == 0 && lane < gamma) ? a.tokens[static_cast<long>(b) * gamma + lane] : -1;
  const int g = request_len(a.lens, gamma, b);
  const float T = request_T(a.temps, a.scalar_T, b);
  const bool greedy = KIND == kGreedyOnly ? true : (KIND == kStochasticOnly ? false : !(T > 0.0f));
  const float c = greedy ? 0.0f : temp_scale(T);
  float ua = 0.0f, us = 0.0f;
  if (!greedy) {
#pragma unroll
    for (int q = 0; q < kSmBatch; ++q) {
      const int e = q * kSmBlock + tid;
      bd[q] = e < nd ? load_one<DT>(db, e) : -INFINITY;
    }
    if (wave == 0 && lane < g) ua = a.u_accept[static_cast<long>(b) * gamma + lane];
    us = a.u_sample[b];
  }
#pragma unroll
  for (int q = 0; q < kSmBatch; ++q) {
    const int e = q * kSmBlock + tid;
    if (e < nt) zs[e] = bt[q];
  }
  if (!greedy) {
#pragma unroll
    for (int q = 0; q < kSmBatch; ++q) {
      const int e = q * kSmBlock + tid;
      if (e < nd) zs[nt + e] = bd[q];
    }
  }
  auto row_needed = [&](int r) { return r <= gamma ? r <= g : (!greedy && r - gamma - 1 < g); };
  __syncthreads();

  // row statistics, one wave per row; a lane takes kSmRun tokens at a time
  // (read together, folded as K1 folds a tile)
  for (int r = wave; r < rows; r += kSmWaves) {
    if (!row_needed(r)) continue;  // uniform per wave
    const float *z = zs + static_cast<long>(r) * V;
    int M = kEmptyM;
    double s = 0.0;
    float mx = -INFINITY;
    int bi = 0x7fffffff;
    for (int v0 = lane; v0 < V; v0 += kSmRun * kWave) {
      float zz[kSmRun];
#pragma unroll
      for (int q = 0; q < kSmRun; ++q) {  // clamped reads, then a select: no branch per token
        const int v = v0 + q * kWave;
        const float zv = z[min(v, V - 1)];
        zz[q] = v < V ? zv : -INFINITY;
      }
      if (!greedy) {
        fold_values<kSmRun>(zz, c, M, s, mx);
      } else {
        // a lane's tokens come in increasing order: a strict > keeps the first
#pragma unroll
        for (int q = 0; q < kSmRun; ++q) {
          const bool take = v0 + q * kWave < V && (bi == 0x7fffffff || zz[q] > mx);
          mx = take ? zz[q] : mx;
          bi = take ? v0 + q * kWave : bi;
        }
      }
    }
    // merged over the wave with DPP: the largest M, every lane's sum rescaled
    // to it exactly (a power of two), then one fp64 sum; greedy: the maximum,
    // then the lowest index holding it
    const float wmx = wave_max_f32(mx);
    if (!greedy) {
      const int Mw = wave_ext_i32<true>(M);
      const double sw = wave_sum(M == kEmptyM ? 0.0 : ldexp(s, M - Mw));
      if (lane == 0) {
        sh_M[r] = Mw;
        sh_s[r] = sw;
        sh_mx[r] = wmx;
      }
    } else {
      const int wbi = wave_ext_i32<false>(mx == wmx ? bi : INT_MAX);
      if (lane == 0) {
        sh_arg[r] = wbi;
        sh_mx[r] = wmx;
      }
    }
  }
  __syncthreads();

  // decision (wave 0): acceptance of each draft and the first rejection
  if (wave == 0) {
    const sv_debug &d = a.dbg;
    const int p = lane;
    bool reject = false;
    if (p < g) {
      if (x < 0 || x >= V) {
        reject = true;  // a draft id outside the vocabulary is rejected, never dereferenced
      } else if (greedy) {
        reject = x != sh_arg[p];
      } else {
        const float zpx = zs[static_cast<long>(p) * V + x];
        const float zqx = zs[static_cast<long>(gamma + 1 + p) * V + x];
        const double cd = static_cast<double>(c);
        const int Mp = sh_M[p], Mq = sh_M[gamma + 1 + p];
        const double sp_ = sh_s[p], sq_ = sh_s[gamma + 1 + p];
        // p/q at x = 2^((zp - zq) c - (Mp - Mq)) * s_q / s_p, in fp64
        const double dd = (static_cast<double>(zpx) - static_cast<double>(zqx)) * cd - static_cast<double>(Mp - Mq);
        const double ratio = exp2(dd) * (sq_ / sp_);
        const double acc = ratio < 1.0 ? ratio : 1.0;
        reject = !(static_cast<double>(ua) < acc);
        const long o = static_cast<long>(b) * gamma + p;
        if (d.p_draft) d.p_draft[o] = exp2(static_cast<double>(zpx) * cd - Mp) / sp_;
        if (d.q_draft) d.q_draft[o] = exp2(static_cast<double>(zqx) * cd - Mq) / sq_;
        if (d.accept_prob) d.accept_prob[o] = acc;
      }
    }
    const unsigned long long rej = __ballot(reject);
    const int k = rej ? (__ffsll(static_cast<long long>(rej)) - 1) : g;
    // row diagnostics of every row read
    for (int r = lane; r < rows; r += kWave) {
      if (!row_needed(r)) continue;
      if (!greedy) {
        if (d.row_max) d.row_max[static_cast<long>(b) * rows + r] = sh_mx[r];
        if (d.row_sum)  // sum_v exp((z_v - max)/T) = s * 2^(M - max c)
          d.row_sum[static_cast<long>(b) * rows + r] =
              sh_s[r] * exp2(static_cast<double>(sh_M[r]) - static_cast<double>(sh_mx[r]) * static_cast<double>(c));
      } else if (d.row_argmax && r <= gamma) {
        d.row_argmax[static_cast<long>(b) * (gamma + 1) + r] = sh_arg[r];
      }
    }
    // outputs; a stochastic request's token at k is drawn below
    if (lane <= gamma) {  // gamma < 64: lane t holds draft t
      const int t = lane;
      int32_t v = -1;
      if (t < k) v = x;
      else if (t == k && greedy) v = sh_arg[k];
      if (t != k || greedy) a.out[static_cast<long>(b) * (gamma + 1) + t] = v;
    }
    if (lane == 0) {
      a.count[b] = k;
      sh_k = k;
    }
  }
  __syncthreads();
  if (greedy) return;  // uniform per workgroup

  // draw at position k: the residual max(0, p_k - q_k) in units of the target
  // row's scale (e_p - r e_q), or p_k for the bonus / a residual of mass zero
  const int k = sh_k;
  const bool useq = k < g;
  const float negMp = -static_cast<float>(sh_M[k]);
  const float negMq = useq ? -static_cast<float>(sh_M[gamma + 1 + k]) : 0.0f;
  const float rr = useq ? static_cast<float>(sh_s[k] / sh_s[gamma + 1 + k]) : 0.0f;
  const float *zp = zs + static_cast<long>(k) * V;
  const float *zq = zs + static_cast<long>(gamma + 1 + k) * V;
  const int C = (V + kSmBlock - 1) / kSmBlock;
  const int v0 = min(tid * C, V), v1 = min(v0 + C, V);
  auto value = [&](int v, bool use_p) -> float {
    const float ep = __builtin_amdgcn_exp2f(fmaf(zp[v], c, negMp));
    if (use_p || !useq) return ep;
    const float eq = __builtin_amdgcn_exp2f(fmaf(zq[v], c, negMq));
    return fmaxf(0.0f, fmaf(-eq, rr, ep));
  };
  // the threads' sums, their block prefix and the total (two passes: the
  // residual, then p when its mass is zero)
  double excl = 0.0, mine = 0.0, Z = 0.0;
  bool use_p = false;
  for (int pass = 0; pass < 2; ++pass) {
    use_p = pass == 1;
    mine = 0.0;
    for (int v = v0; v < v1; ++v) mine += static_cast<double>(value(v, use_p));
    const double incl = wave_scan(mine, lane);
    if (lane == kWave - 1) sh_wtot[wave] = incl;
    __syncthreads();
    double before = 0.0;
    Z = 0.0;
    for (int w = 0; w < kSmWaves; ++w) {
      const double t = sh_wtot[w];
      if (w < wave) before += t;
      Z += t;
    }
    excl = before + (incl - mine);
    if (Z > 0.0 || !useq) break;  // uniform: every thread read the same totals
    __syncthreads();              // sh_wtot is rewritten by the second pass
  }
  const double target = static_cast<double>(us) * Z;
  // the first thread whose range crosses u*Z (tokens with mass only), found
  // by every wave from the same wave totals: the crossing wave, then its
  // lane by a ballot; if rounding leaves u*Z past the end, the last thread
  // with mass
  int cw = -1, lw = -1;
  {
    double run = 0.0;
    for (int w = 0; w < kSmWaves; ++w) {
      const double t = sh_wtot[w];
      if (t > 0.0) {
        if (cw < 0 && run + t > target) cw = w;
        lw = w;
      }
      run += t;
    }
  }
  const bool past_end = cw < 0;
  if (past_end) cw = lw < 0 ? 0 : lw;
  if (wave != cw) return;  // uniform per wave
  const unsigned long long hit = __ballot(mine > 0.0 && excl + mine > target);
  const unsigned long long has = __ballot(mine > 0.0);
  const int L = (!past_end && hit) ? __ffsll(static_cast<long long>(hit)) - 1
                                   : (has ? 63 - __clzll(static_cast<long long>(has)) : 0);
  if (lane == L) {
    double acc = excl;
    int tok = -1, lastm = -1;
    for (int v = v0; v < v1; ++v) {
      const float w = value(v, use_p);
      if (w > 0.0f) {
        lastm = v;
        acc += static_cast<double>(w);
        if (tok < 0 && target < acc) tok = v;
      }
    }
    if (tok < 0) tok = lastm >= 0 ? lastm : v0;
    a.out[static_cast<long>(b) * (gamma + 1) + k] = tok;
    if (a.dbg.residual_mass) a.dbg.residual_mass[b] = Z / sh_s[k];
  }
}

// ================================================================== draft-side sampler
// One token per row of softmax(z/T), in two kernels.
//   S1 k_sample_stats: kSBlock-thread workgroups, several per row; each wave
//      takes 2048-token sub-chunks of a row and records (M_j, s_j =
//      sum 2^(z c - M_j)), M_j = ceil(max_j * c) the sub-chunk's own integer
//      reference, or for a greedy row its (max, lowest index).
//   S2 k_sample_pick: one wave per row.  The row's masses are
//      m_j = s_j * 2^(M_j - M) (exact), the sub-chunk holding u*Z is found by
//      a scan, and only that sub-chunk is read again.
constexpr int kSBlock = 256;
constexpr int kSWaves = kSBlock / kWave;
constexpr long kSTargetWaves = 4096;  // waves of S1 (16 per CU)

struct alignas(16) SubRecord {
  double s;  // sum 2^(z c - M_j) over the sub-chunk (stochastic)
  float mx;  // the sub-chunk's maximum (greedy)
  int mi;    // M_j (stochastic) or the maximum's lowest index (greedy)
};


// S1: workgroup g of row r (SG workgroups per row); wave w takes sub-chunks
// g * kSWaves + w, then every SG * kSWaves further.
template <int DT>
__global__ __launch_bounds__(kSBlock) void k_sample_stats(const void *__restrict__ logits,
                                                          const float *__restrict__ temps, float scalar_T, int V,
                                                          int NSUB, int SG, SubRecord *__restrict__ rec) {
  constexpr int kN = kLaneElems / Elem<DT>::kVec;
  const int r = blockIdx.x / SG, g = blockIdx.x - r * SG;
  const int lane = threadIdx.x & (kWave - 1), wave = threadIdx.x / kWave;
  const float T = temps ? temps[r] : scalar_T;
  const bool greedy = !(T > 0.0f);
  const float c = greedy ? 0.0f : temp_scale(T);
  const char *row = static_cast<const char *>(logits) + static_cast<long>(r) * V * Elem<DT>::kBytes;
  const bool aligned = (reinterpret_cast<uintptr_t>(row) & 15u) == 0;
  for (int sub = g * kSWaves + wave; sub < NSUB; sub += SG * kSWaves) {
    u32x4 raw[kN];
    load_lane_raw<DT>(row, aligned, static_cast<long>(sub) * kSub, lane, V, raw);
    SubRecord rc;
    if (!greedy) {
      float lmx = -INFINITY;
#pragma unroll
      for (int q = 0; q < kN; ++q) {
        float x[Elem<DT>::kVec];
        widen_vec<DT>(raw[q], x);
#pragma unroll
        for (int e = 0; e < Elem<DT>::kVec; ++e) lmx = fmaxf(lmx, x[e]);
      }
      const float wmx = wave_max_f32(lmx);
      int M = kEmptyM;
      double sw = 0.0;
      if (wmx > -INFINITY) {
        const float Mf = ceilf(wmx * c);
        M = static_cast<int>(Mf);
        float acc[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) acc[e] = 0.0f;
#pragma unroll
        for (int q = 0; q < kN; ++q) {
          float x[Elem<DT>::kVec];
          widen_vec<DT>(raw[q], x);
#pragma unroll
          for (int e = 0; e < Elem<DT>::kVec; ++e)
            acc[(q * Elem<DT>::kVec + e) & 7] += __builtin_amdgcn_exp2f(fmaf(x[e], c, -Mf));
        }
        const float ls = ((acc[0] + acc[1]) + (acc[2] + acc[3])) + ((acc[4] + acc[5]) + (acc[6] + acc[7]));
        sw = wave_sum(static_cast<double>(ls));
      }
      rc.s = sw;
      rc.mx = wmx;
      rc.mi = M;
    } else {
      float bv = -INFINITY;
      int bi = 0x7fffffff;
#pragma unroll
      for (int q = 0; q < kN; ++q) {  // the lane's tokens in increasing index order
        float x[Elem<DT>::kVec];
        widen_vec<DT>(raw[q], x);
        const long e0 = static_cast<long>(sub) * kSub + static_cast<long>(q * kWave + lane) * Elem<DT>::kVec;
#pragma unroll
        for (int e = 0; e < Elem<DT>::kVec; ++e) {
          if (e0 + e < V && (x[e] > bv || bi == 0x7fffffff)) {
            bv = x[e];
            bi = static_cast<int>(e0 + e);
          }
        }
      }
      const float vw = wave_max_f32(bv);  // then the lowest index holding it (DPP)
      rc.s = 0.0;
      rc.mx = vw;
      rc.mi = wave_ext_i32<false>(bv == vw ? bi : INT_MAX);
    }
    if (lane == 0) rec[static_cast<long>(r) * NSUB + sub] = rc;
  }
}

// S2: one wave per row.
template <int DT>
__global__ __launch_bounds__(kWave) void k_sample_pick(const void *__restrict__ logits, const float *__restrict__ u,
                                                       const float *__restrict__ temps, float scalar_T, int V,
                                                       int NSUB, const SubRecord *__restrict__ rec,
                                                       int32_t *__restrict__ tokens) {
  const int r = blockIdx.x;
  const int lane = threadIdx.x;
  const float T = temps ? temps[r] : scalar_T;
  const bool greedy = !(T > 0.0f);
  const float c = greedy ? 0.0f : temp_scale(T);
  const char *row = static_cast<const char *>(logits) + static_cast<long>(r) * V * Elem<DT>::kBytes;
  const bool aligned = (reinterpret_cast<uintptr_t>(row) & 15u) == 0;
  const SubRecord *rr = rec + static_cast<long>(r) * NSUB;

  if (greedy) {
    float bv = -INFINITY;
    int bi = 0x7fffffff;
    for (int j = lane; j < NSUB; j += kWave) merge_arg(bv, bi, rr[j].mx, rr[j].mi);
    const float vw = wave_max_f32(bv);  // then the lowest index holding it (DPP)
    const int iw = wave_ext_i32<false>(bv == vw ? bi : INT_MAX);
    if (lane == 0) tokens[r] = iw;
    return;
  }
  // the row's reference exponent and the sub-chunk masses m_j = s_j 2^(M_j - M)
  int M = kEmptyM;
  for (int j = lane; j < NSUB; j += kWave) M = max(M, rr[j].mi);
  M = wave_ext_i32<true>(M);
  auto mass = [&](int j) { return j < NSUB ? ldexp(rr[j].s, rr[j].mi - M) : 0.0; };
  double Z = 0.0;
  for (int base = 0; base < NSUB; base += kWave) Z += wave_sum(mass(base + lane));
  const double target_mass = static_cast<double>(u[r]) * Z;
  int sub = -1;
  double base_mass = 0.0, run = 0.0;
  for (int base = 0; base < NSUB; base += kWave) {
    const int j = base + lane;
    const double v = mass(j);
    const double incl = wave_scan(v, lane);
    const unsigned long long hit = __ballot(j < NSUB && v > 0.0 && run + incl > target_mass);
    if (hit) {
      const int L = __ffsll(static_cast<long long>(hit)) - 1;
      sub = base + L;
      base_mass = run + lane_value(incl - v, L);
      break;
    }
    run += lane_value(incl, kWave - 1);
  }
  if (sub < 0) {  // rounding left u*Z at the very end: the last sub-chunk with mass
    run = 0.0;
    for (int base = 0; base < NSUB; base += kWave) {
      const int j = base + lane;
      const double v = mass(j);
      const double incl = wave_scan(v, lane);
      const unsigned long long has = __ballot(j < NSUB && v > 0.0);
      if (has) {
        const int L = 63 - __clzll(static_cast<long long>(has));
        sub = base + L;
        base_mass = run + lane_value(incl - v, L);
      }
      run += lane_value(incl, kWave - 1);
    }
    if (sub < 0) {
      sub = 0;
      base_mass = 0.0;
    }
  }
  // the token inside the sub-chunk: the same per-token values as the first
  // pass (reference M_sub), rescaled exactly to the row reference
  const int Ms = rr[sub].mi;
  const long first = static_cast<long>(sub) * kSub + static_cast<long>(lane) * kLaneElems;
  float z[kLaneElems];
#pragma unroll
  for (int q = 0; q < kLaneElems / Elem<DT>::kVec; ++q)
    load_vec_guarded<DT>(row, aligned, first + q * Elem<DT>::kVec, V, z + q * Elem<DT>::kVec);
  double vals[kLaneElems];
  double lsum = 0.0;
#pragma unroll
  for (int e = 0; e < kLaneElems; ++e) {
    vals[e] = ldexp(static_cast<double>(__builtin_amdgcn_exp2f(fmaf(z[e], c, -static_cast<float>(Ms)))), Ms - M);
    lsum += vals[e];
  }
  const double incl = wave_scan(lsum, lane);
  double acc = base_mass + (incl - lsum);
  int cand = -1, last_pos = -1;
#pragma unroll
  for (int e = 0; e < kLaneElems; ++e) {
    if (vals[e] > 0.0) {
      last_pos = e;
      acc += vals[e];
      if (cand < 0 && target_mass < acc) cand = e;
    }
  }
  const unsigned long long props = __ballot(cand >= 0);
  if (props) {
    if (lane == __ffsll(static_cast<long long>(props)) - 1) tokens[r] = static_cast<int>(first + cand);
  } else {
    const unsigned long long has = __ballot(last_pos >= 0);
    const int L = has ? 63 - __clzll(static_cast<long long>(has)) : 0;
    if (lane == L) tokens[r] = static_cast<int>(first + (last_pos >= 0 ? last_pos : 0));
  }
}

// ================================================================== host side
struct Plan {
  int rows, NS, chunk_vecs, NSUB, SPW, NW;
  long k1_groups, k3_groups;
  long k1_groups_g;  // K1 grid when every request is greedy (the gamma + 1 target rows only)
  size_t part_off, zx_off, sel_off, sums_off, fst_off, total;
  // filtered calls: buffers of the filter kernels after `total`
  size_t ncand_off, cand_off, dcount_off, ftotal;
};

size_t align_up(size_t x) { return (x + kAlign - 1) / kAlign * kAlign; }

constexpr int kK1U = 8;                 // 16-byte vectors per thread per K1 tile
constexpr long kK1TargetGroups = 4224;  // about 16 workgroups per CU on 256 CUs (a sweep)
// Unfiltered verify calls: about 1408 workgroups, at least two chunks per row.
// B = 64, gamma = 5, V = 128256 bf16 (704 rows of 8 tiles): 2 chunks per row (1408 workgroups) 45.6-46.2
// us per call against 46.6-47.8 with 4 (2816); the ragged B = 128 batch (1920
// row slots of 10 tiles) keeps 2 chunks per row (1 measured 76.8-77.0 us
// against 75.0).
constexpr long kK1VerifyTargetGroups = 1408;
// Uniform greedy batches (max and index only, 90 registers): fewer, longer
// workgroups.  B = 64, gamma = 5, V = 128256 bf16, greedy (384 target rows of 8 tiles): 768 workgroups
// (2 chunks per row) 20.7-21.2 us per call, 1152 21.8, 1536 21.2-21.5, 3072
// about 21.8.
constexpr long kK1GreedyTargetGroups = 768;

// kind: the K1 grid the chunks are sized for (kPlanVerify and kPlanGreedy: an
// unfiltered verify call, stochastic or mixed / a uniform greedy batch, whose K1
// grid covers the gamma + 1 target rows of each request only).
enum { kPlanDefault = 0, kPlanVerify = 1, kPlanGreedy = 2 };
bool make_plan(int B, int gamma, int V, int dtype, Plan *P, int gamma_limit = SV_GAMMA_MAX,
               int kind = kPlanDefault) {
  const bool greedy_only = kind == kPlanGreedy;
  if (B < 1 || gamma < 0 || gamma > gamma_limit || V < 1) return false;
  if (dtype != SV_F32 && dtype != SV_BF16) return false;
  const int vec = dtype == SV_BF16 ? 8 : 4;
  P->rows = 2 * gamma + 1;
  const long slots = static_cast<long>(B) * P->rows;
  // split each row into NS chunks of whole K1 tiles: enough workgroups to fill
  // the chip, no chunk shorter than one tile.  Chunk lengths are whole tiles,
  // so that only the row's last chunk ends in a partial (masked) tile.
  const long vecs = (V + vec - 1) / vec;
  const long tile = static_cast<long>(kK1U) * kBlock;
  const long tiles_per_row = (vecs + tile - 1) / tile;
  const long plan_slots = greedy_only ? static_cast<long>(B) * (gamma + 1) : slots;
  const long target = greedy_only ? kK1GreedyTargetGroups
                                  : (kind == kPlanVerify ? kK1VerifyTargetGroups : kK1TargetGroups);
  long NS = (target + plan_slots / 2) / plan_slots;
  if (NS < (kind == kPlanVerify ? 2 : 1)) NS = kind == kPlanVerify ? 2 : 1;
  if (NS > tiles_per_row) NS = tiles_per_row;
  const long tiles_per_chunk = (tiles_per_row + NS - 1) / NS;
  P->chunk_vecs = static_cast<int>(tiles_per_chunk * tile);
  NS = (tiles_per_row + tiles_per_chunk - 1) / tiles_per_chunk;  // every chunk non-empty
  P->NS = static_cast<int>(NS);
  P->k1_groups = slots * NS;
  // greedy-only batches: the grid covers the target rows only
  P->k1_groups_g = static_cast<long>(B) * (gamma + 1) * NS;
  P->NSUB = (V + kSub - 1) / kSub;
  // sub-chunks per wave in the mass pass: one (two, the second prefetched,
  // measured slower at B = 64 and at B = 128)
  P->SPW = 1;
  P->NW = (P->NSUB + kWaves * P->SPW - 1) / (kWaves * P->SPW);
  P->k3_groups = static_cast<long>(B) * P->NW;
  // 1-D grids: work-items per launch must stay below 2^32
  const long max_groups = (1L << 32) / kBlock - 1;
  if (P->k1_groups > max_groups || P->k3_groups > max_groups || P->k1_groups_g > max_groups) return false;
  size_t off = 0;
  P->part_off = off;
  off = align_up(off + sizeof(Partial) * static_cast<size_t>(P->k1_groups));
  P->zx_off = off;
  off = align_up(off + sizeof(float) * static_cast<size_t>(slots));
  P->sel_off = off;
  off = align_up(off + sizeof(SelParams) * static_cast<size_t>(B));
  P->sums_off = off;
  off = align_up(off + sizeof(SubSums) * static_cast<size_t>(B) * P->NSUB);
  P->fst_off = off;
  off = align_up(off + sizeof(FilterStats) * static_cast<size_t>(slots));
  P->total = off;
  P->ncand_off = off;
  off = align_up(off + sizeof(unsigned) * static_cast<size_t>(slots));
  P->cand_off = off;
  off = align_up(off + sizeof(unsigned) * static_cast<size_t>(slots) * kGCap);
  P->dcount_off = off;
  off = align_up(off + sizeof(unsigned) * static_cast<size_t>(P->k1_groups) * (kDeep + 1));
  P->ftotal = off;
  return true;
}

// K1 launch; with an event pair the dispatch itself is timestamped (the
// events bracket the kernel's execution, as a kernel trace does).
template <int DT, int KIND>
hipError_t launch_k1_kind(const void *target, const void *draft, const int32_t *tokens, const float *temps,
                          float scalar_T, const int32_t *lens, int gamma, int V, const Plan &P,
                          Partial *part, float *zx, hipStream_t st, hipEvent_t ev0, hipEvent_t ev1,
                          unsigned *row_counter, unsigned long long *req_words, int req_words_n) {
  const bool g = KIND == kGreedyOnly;
  const dim3 grid(static_cast<unsigned>(g ? P.k1_groups_g : P.k1_groups)), block(kBlock);
  const int grows = g ? gamma + 1 : P.rows;
  if (ev0 && ev1) {
    hipExtLaunchKernelGGL((k1_row_stats<DT, kK1U, KIND>), grid, block, 0, st, ev0, ev1, 0, target, draft,
                          tokens, temps, scalar_T, lens, gamma, V, P.NS, P.chunk_vecs, grows, part, zx, row_counter,
                          req_words, req_words_n);
  } else {
    hipLaunchKernelGGL((k1_row_stats<DT, kK1U, KIND>), grid, block, 0, st, target, draft, tokens, temps,
                       scalar_T, lens, gamma, V, P.NS, P.chunk_vecs, grows, part, zx, row_counter, req_words,
                       req_words_n);
  }
  return hipGetLastError();
}

template <int DT>
hipError_t launch_k1(const void *target, const void *draft, const int32_t *tokens, const float *temps,
                     float scalar_T, const int32_t *lens, int gamma, int V, const Plan &P, Partial *part,
                     float *zx, hipStream_t st, hipEvent_t ev0, hipEvent_t ev1,
                     unsigned *row_counter = nullptr, unsigned long long *req_words = nullptr,
                     int req_words_n = 0) {
  if (temps)
    return launch_k1_kind<DT, kMixed>(target, draft, tokens, temps, scalar_T, lens, gamma, V, P, part, zx,
                                      st, ev0, ev1, row_counter, req_words, req_words_n);
  if (scalar_T > 0.0f)
    return launch_k1_kind<DT, kStochasticOnly>(target, draft, tokens, temps, scalar_T, lens, gamma, V, P,
                                               part, zx, st, ev0, ev1, row_counter, req_words, req_words_n);
  return launch_k1_kind<DT, kGreedyOnly>(target, draft, tokens, temps, scalar_T, lens, gamma, V, P, part, zx,
                                         st, ev0, ev1, row_counter, req_words, req_words_n);
}

// fractional bits of the filter's fixed-point masses: V * 2^(fs + 1) <= 2^62
int filter_frac_bits(int V) {
  int l = 0;
  while ((1L << l) < V) ++l;
  return 61 - l;
}

template <int DT>
int run(const void *target, const void *draft, const int32_t *tokens, const float *u_accept,
        const float *u_sample, const float *temps, float scalar_T, bool all_greedy,
        const int32_t *lens, const int32_t *topk, const float *topp, int B, int gamma, int V,
        int32_t *count, int32_t *out, void *ws, const Plan &P, hipStream_t st, const sv_debug *dbgp) {
  char *base = static_cast<char *>(ws);
  Partial *part = reinterpret_cast<Partial *>(base + P.part_off);
  float *zx = reinterpret_cast<float *>(base + P.zx_off);
  SelParams *sel = reinterpret_cast<SelParams *>(base + P.sel_off);
  SubSums *sums = reinterpret_cast<SubSums *>(base + P.sums_off);
  FilterStats *fst = (topk || topp) ? reinterpret_cast<FilterStats *>(base + P.fst_off) : nullptr;
  sv_debug dbg;
  memset(&dbg, 0, sizeof dbg);
  if (dbgp) dbg = *dbgp;
  unsigned *ncand = fst ? reinterpret_cast<unsigned *>(base + P.ncand_off) : nullptr;
  // K2 also draws when workgroup 0 can hold the request's sub-chunk masses;
  // K1 then clears the hand-over words (the sub-chunk mass array)
  const bool sel2 = !all_greedy && P.NSUB <= kSelMaxSub;
  // every workgroup waits for its request's masses only when the whole grid is
  // resident at once (K2's registers allow 4 workgroups per CU for bf16 rows,
  // 2 for fp32; 256 CUs).  On the ragged B = 128 batch (2432 workgroups) the
  // waiting workgroups held back the later ones: 79.9 us per call against
  // 76.5 with workgroup 0 drawing; B = 64, V = 128256 (1024) 46.1 against 46.4.
  const bool owner = static_cast<long>(B) * P.NW <= (DT == SV_BF16 ? 1024L : 512L);
  unsigned long long *words = sel2 ? reinterpret_cast<unsigned long long *>(sums) : nullptr;
  hipError_t e = launch_k1<DT>(target, draft, tokens, temps, scalar_T, lens, gamma, V, P, part, zx, st,
                               static_cast<hipEvent_t>(dbg.k1_events[0]),
                               static_cast<hipEvent_t>(dbg.k1_events[1]), ncand, words, sel2 ? 2 * P.NSUB : 0);
  if (e != hipSuccess) return SV_EHIP;
  if (fst) {
    FilterWork fw;
    fw.ncand = ncand;
    fw.cand = reinterpret_cast<unsigned *>(base + P.cand_off);
    fw.dcount = reinterpret_cast<unsigned *>(base + P.dcount_off);
    const int fs = filter_frac_bits(V);
    const dim3 cgrid(static_cast<unsigned>(P.k1_groups)), rgrid(static_cast<unsigned>(static_cast<long>(B) * P.rows));
    hipLaunchKernelGGL((k_filter_capture<DT>), cgrid, dim3(kLBlock), 0, st, target, draft, temps, lens, topk, topp,
                       gamma, V, P.NS, P.chunk_vecs, part, fw);
    if (hipGetLastError() != hipSuccess) return SV_EHIP;
    // the deeper-window counts only concern top-k requests
    if (topk)
      hipLaunchKernelGGL((k_filter_deep_count<DT>), cgrid, dim3(kLBlock), 0, st, target, draft, temps, lens, topk,
                         topp, gamma, V, P.NS, P.chunk_vecs, part, fw);
    hipLaunchKernelGGL((k_filter_resolve<DT>), rgrid, dim3(kFBlock), 0, st, target, draft, temps, lens, topk, topp,
                       gamma, V, P.NS, fs, part, fw, fst);
    hipLaunchKernelGGL((k_filter_general<DT>), rgrid, dim3(kFBlock), 0, st, target, draft, temps, lens, topk, topp,
                       gamma, V, P.NS, fs, part, fst);
    if (hipGetLastError() != hipSuccess) return SV_EHIP;
  }
  // greedy-only batches need the decision alone: one workgroup per request
  const int nw = all_greedy ? 1 : P.NW;
  const dim3 g2(static_cast<unsigned>(static_cast<long>(B) * nw));
#define SV_K2(FILT, SEL)                                                                                  \
  hipLaunchKernelGGL((k2_decide_mass<DT, FILT, SEL>), g2, dim3(kBlock), 0, st, target, draft, tokens, u_accept, \
                     temps, scalar_T, lens, gamma, V, P.NS, P.NSUB, nw, P.SPW, part, zx, topk, topp, fst, count,  \
                     out, sel, sums, u_sample, owner, dbg)
  if (fst) {
    if (sel2) SV_K2(true, true);
    else SV_K2(true, false);
  } else {
    if (sel2) SV_K2(false, true);
    else SV_K2(false, false);
  }
#undef SV_K2
  if (hipGetLastError() != hipSuccess) return SV_EHIP;
  if (!all_greedy && !sel2) {
    if (fst)
      hipLaunchKernelGGL((k3_select<DT, true>), dim3(B), dim3(kBlock), 0, st, target, draft, u_sample, gamma,
                         V, P.NSUB, sel, sums, out, dbg.residual_mass);
    else
      hipLaunchKernelGGL((k3_select<DT, false>), dim3(B), dim3(kBlock), 0, st, target, draft, u_sample, gamma,
                         V, P.NSUB, sel, sums, out, dbg.residual_mass);
    if (hipGetLastError() != hipSuccess) return SV_EHIP;
  }
  return SV_OK;
}

// ------------------------------------------------------------------ small problems
// One workgroup per request when a request's rows hold at most kSmElems logits.
bool small_problem(int gamma, int V) { return static_cast<long>(2 * gamma + 1) * V <= kSmElems; }

template <int DT>
int run_small(const void *target, const void *draft, const int32_t *tokens, const float *u_accept,
              const float *u_sample, const float *temps, float scalar_T, const int32_t *lens, int B, int gamma,
              int V, int32_t *count, int32_t *out, hipStream_t st, const sv_debug *dbgp) {
  SmallArgs sa;
  memset(&sa, 0, sizeof sa);
  if (dbgp) sa.dbg = *dbgp;
  sa.target = target;
  sa.draft = draft;
  sa.tokens = tokens;
  sa.u_accept = u_accept;
  sa.u_sample = u_sample;
  sa.temps = temps;
  sa.scalar_T = scalar_T;
  sa.lens = lens;
  sa.gamma = gamma;
  sa.V = V;
  sa.count = count;
  sa.out = out;
  const size_t lds = sizeof(float) * static_cast<size_t>(2 * gamma + 1) * V;
  const hipEvent_t ev0 = static_cast<hipEvent_t>(sa.dbg.k1_events[0]), ev1 = static_cast<hipEvent_t>(sa.dbg.k1_events[1]);
#define SV_SMALL(KIND)                                                                                        \
  do {                                                                                                        \
    if (ev0 && ev1)                                                                                           \
      hipExtLaunchKernelGGL((k_small_verify<DT, KIND>), dim3(B), dim3(kSmBlock), lds, st, ev0, ev1, 0, sa);   \
    else                                                                                                      \
      hipLaunchKernelGGL((k_small_verify<DT, KIND>), dim3(B), dim3(kSmBlock), lds, st, sa);                   \
  } while (0)
  if (temps) SV_SMALL(kMixed);
  else if (scalar_T > 0.0f) SV_SMALL(kStochasticOnly);
  else SV_SMALL(kGreedyOnly);
#undef SV_SMALL
  return hipGetLastError() == hipSuccess ? SV_OK : SV_EHIP;
}

int dispatch(const void *target, const void *draft, const int32_t *tokens, const float *u_accept,
             const float *u_sample, const float *temps, float scalar_T, bool all_greedy,
             const int32_t *lens, const int32_t *topk, const float *topp, int B, int gamma, int V,
             int dtype, int32_t *count, int32_t *out, void *ws, size_t ws_bytes, void *stream,
             const sv_debug *dbg) {
  Plan P;
  const int plan_kind = (topk || topp) ? kPlanDefault : ((all_greedy && !temps) ? kPlanGreedy : kPlanVerify);
  if (!make_plan(B, gamma, V, dtype, &P, SV_GAMMA_MAX, plan_kind)) return SV_EINVAL;
  if ((topk || topp) &&
      (!temps || V > SV_FILTER_MAX_V || static_cast<long>(B) * P.rows * kFBlock >= (1L << 32)))
    return SV_EINVAL;
  if (!target || !u_sample || !count || !out) return SV_EINVAL;
  if (gamma > 0 && !tokens) return SV_EINVAL;
  if (gamma > 0 && !all_greedy && (!draft || !u_accept)) return SV_EINVAL;
  const size_t need = (topk || topp) ? P.ftotal : P.total;
  if (!ws || (reinterpret_cast<uintptr_t>(ws) % kAlign) != 0 || ws_bytes < need) return SV_EWORKSPACE;
  if (dbg && ((dbg->k1_events[0] == nullptr) != (dbg->k1_events[1] == nullptr))) return SV_EINVAL;
  hipStream_t st = static_cast<hipStream_t>(stream);
  if (!(topk || topp) && small_problem(gamma, V)) {
    if (dtype == SV_BF16)
      return run_small<SV_BF16>(target, draft, tokens, u_accept, u_sample, temps, scalar_T, lens, B, gamma, V,
                                count, out, st, dbg);
    return run_small<SV_F32>(target, draft, tokens, u_accept, u_sample, temps, scalar_T, lens, B, gamma, V, count,
                             out, st, dbg);
  }
  if (dtype == SV_BF16)
    return run<SV_BF16>(target, draft, tokens, u_accept, u_sample, temps, scalar_T, all_greedy, lens, topk,
                        topp, B, gamma, V, count, out, ws, P, st, dbg);
  return run<SV_F32>(target, draft, tokens, u_accept, u_sample, temps, scalar_T, all_greedy, lens, topk, topp,
                     B, gamma, V, count, out, ws, P, st, dbg);
}

constexpr int kMaxDevices = 64;

// ------------------------------------------------------------------ tree walk
// The tree call's workspace: the linear plan, then two copies of each
// request's sub-chunk mass words and of its per-wave statistics words, the
// walk's error word (these three zeroed before each walk, by K1 or by a
// clear), and a spare block the walk's unused row-slice loads read.
struct TreeLayout {
  size_t sub_off, stat_off, err_off, spare_off, total;
  int Wmax;  // waves a team can have
};

TreeLayout tree_layout(int B, const Plan &P) {
  TreeLayout L;
  L.Wmax = (P.NSUB + kTWaves - 1) / kTWaves * kTWaves;
  size_t off = P.total;
  L.sub_off = off;  // mass words, then statistics words, then the error word: one region to clear
  off = align_up(off + sizeof(unsigned long long) * 2 * static_cast<size_t>(B) * P.NSUB);
  L.stat_off = off;
  off = align_up(off + sizeof(unsigned long long) * 2 * static_cast<size_t>(B) * L.Wmax * 4);
  L.err_off = off;
  off = align_up(off + sizeof(unsigned));
  L.spare_off = off;  // a block the walk's unused row-slice loads read (contents never used)
  off = align_up(off + sizeof(float) * kSub);
  L.total = off;
  return L;
}

// Workgroups per request for the tree walk: enough for one 2048-token sub-chunk
// per wave, as long as the whole grid stays within half of the workgroups the
// device holds at once (the team's workgroups wait for each other after every
// pass, so they must all be resident); large batches walk with one workgroup
// per request.
template <int DT, bool OD>
int tree_team_size(int B, int NSUB) {
  static int cache[kMaxDevices];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return 1;
  if (!cache[dev]) {
    int cus = 0, per = 0;
    if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
        hipOccupancyMaxActiveBlocksPerMultiprocessor(&per, k_tree_walk<DT, OD>, kTBlock, 0) != hipSuccess)
      return 1;
    cache[dev] = max(1, cus * per / 2);
  }
  const int want = (NSUB + kTWaves - 1) / kTWaves;
  const int room = cache[dev] / B;
  return max(1, min(want, room));
}

// ------------------------------------------------------------------ built-in scratch
// Scratch of spec_verify_noalloc: one array per GPU (each GPU that loads the
// code object holds its own copy).  In host code `scratch` only names the
// symbol; its device address comes from hipGetSymbolAddress, looked up once per
// device with that device current, and only that address is passed to kernels.
static __device__ __align__(256) unsigned char scratch[SV_NOALLOC_SCRATCH_BYTES];

std::mutex g_scratch_mutex;
void *g_scratch_ptr[kMaxDevices];

// Device address of the current device's scratch array (nullptr on failure).
void *scratch_address() {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return nullptr;
  std::lock_guard<std::mutex> lock(g_scratch_mutex);
  if (!g_scratch_ptr[dev]) {
    void *ptr = nullptr;
    if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)) != hipSuccess || !ptr) return nullptr;
    g_scratch_ptr[dev] = ptr;
  }
  return g_scratch_ptr[dev];
}

// The tree walk, after K1 over every position's rows (statistics from K1) or
// alone (OD: statistics on demand, the exchange words already cleared).
template <int DT, bool OD>
int launch_tree(const void *target, const void *draft, const int32_t *parent, const int32_t *tokens,
                const int32_t *num_nodes, const float *u_accept, const float *u_sample, const float *temps, int B,
                int max_nodes, int V, const Plan &P, const TreeLayout &L, char *base, int32_t *count, int32_t *out,
                int32_t *out_nodes, hipStream_t st) {
  Partial *part = reinterpret_cast<Partial *>(base + P.part_off);
  float *zx = reinterpret_cast<float *>(base + P.zx_off);
  unsigned long long *tsub = reinterpret_cast<unsigned long long *>(base + L.sub_off);
  unsigned long long *tstat = reinterpret_cast<unsigned long long *>(base + L.stat_off);
  unsigned *terr = reinterpret_cast<unsigned *>(base + L.err_off);
  if constexpr (!OD) {
    if (launch_k1<DT>(target, draft, tokens, temps, 0.0f, num_nodes, max_nodes, V, P, part, zx, st, nullptr, nullptr,
                      nullptr, tsub, 2 * P.NSUB) != hipSuccess)
      return SV_EHIP;
  }
  const int NW = tree_team_size<DT, OD>(B, P.NSUB);
  hipLaunchKernelGGL((k_tree_walk<DT, OD>), dim3(static_cast<unsigned>(static_cast<long>(B) * NW)), dim3(kTBlock),
                     0, st, target, draft, parent, tokens, num_nodes, u_accept, u_sample, temps, max_nodes, V, P.NS,
                     part, count, out, out_nodes, NW, tsub, terr, base + L.spare_off, tstat, L.Wmax);
  return hipGetLastError() == hipSuccess ? SV_OK : SV_EHIP;
}

// Workspace of an unfiltered verify call: the largest over the K1 grids that
// dispatch may choose for it (0 for an invalid shape).
size_t verify_total(int B, int gamma, int V, int dtype) {
  size_t total = 0;
  for (int kind : {kPlanDefault, kPlanVerify, kPlanGreedy}) {
    Plan P;
    if (!make_plan(B, gamma, V, dtype, &P, SV_GAMMA_MAX, kind)) return 0;
    if (P.total > total) total = P.total;
  }
  return total;
}

}  // namespace

// ================================================================== C ABI
extern "C" {

size_t spec_verify_workspace_bytes(int B, int gamma, int V, int dtype) {
  return verify_total(B, gamma, V, dtype);
}

int spec_verify(const void *target_logits, const void *draft_logits, const int32_t *draft_tokens,
                const float *u_accept, const float *u_sample, float temperature, int B, int gamma,
                int V, int dtype, int32_t *accepted_count, int32_t *out_tokens, void *workspace,
                size_t workspace_bytes, void *stream) {
  if (!(temperature >= 0.0f) || isinf(temperature)) return SV_EINVAL;
  return dispatch(target_logits, draft_logits, draft_tokens, u_accept, u_sample, nullptr, temperature,
                  temperature == 0.0f, nullptr, nullptr, nullptr, B, gamma, V, dtype, accepted_count,
                  out_tokens, workspace, workspace_bytes, stream, nullptr);
}

int spec_verify_dbg(const void *target_logits, const void *draft_logits, const int32_t *draft_tokens,
                    const float *u_accept, const float *u_sample, float temperature, int B, int gamma,
                    int V, int dtype, int32_t *accepted_count, int32_t *out_tokens, void *workspace,
                    size_t workspace_bytes, void *stream, const sv_debug *dbg) {
  if (!(temperature >= 0.0f) || isinf(temperature)) return SV_EINVAL;
  return dispatch(target_logits, draft_logits, draft_tokens, u_accept, u_sample, nullptr, temperature,
                  temperature == 0.0f, nullptr, nullptr, nullptr, B, gamma, V, dtype, accepted_count,
                  out_tokens, workspace, workspace_bytes, stream, dbg);
}

int spec_verify_noalloc(const void *target_logits, const void *draft_logits, const int32_t *draft_tokens,
                        const float *u_accept, const float *u_sample, float temperature, int B, int gamma,
                        int V, int dtype, int32_t *accepted_count, int32_t *out_tokens, void *stream) {
  if (!(temperature >= 0.0f) || isinf(temperature)) return SV_EINVAL;
  const size_t total = verify_total(B, gamma, V, dtype);
  if (total == 0) return SV_EINVAL;
  if (total > static_cast<size_t>(SV_NOALLOC_SCRATCH_BYTES)) return SV_ESCRATCH;
  void *ws = scratch_address();
  if (!ws) return SV_EHIP;
  return dispatch(target_logits, draft_logits, draft_tokens, u_accept, u_sample, nullptr, temperature,
                  temperature == 0.0f, nullptr, nullptr, nullptr, B, gamma, V, dtype, accepted_count,
                  out_tokens, ws, SV_NOALLOC_SCRATCH_BYTES, stream, nullptr);
}

int spec_verify_ex(const void *target_logits, const void *draft_logits, const int32_t *draft_tokens,
                   const float *u_accept, const float *u_sample, const float *temperature,
                   const int32_t *draft_lens, int B, int gamma, int V, int dtype,
                   int32_t *accepted_count, int32_t *out_tokens, void *workspace,
                   size_t workspace_bytes, void *stream, const sv_debug *dbg) {
  if (!temperature) return SV_EINVAL;
  return dispatch(target_logits, draft_logits, draft_tokens, u_accept, u_sample, temperature, 0.0f,
                  false, draft_lens, nullptr, nullptr, B, gamma, V, dtype, accepted_count, out_tokens,
                  workspace, workspace_bytes, stream, dbg);
}

size_t spec_verify_filtered_workspace_bytes(int B, int gamma, int V, int dtype) {
  Plan P;
  if (!make_plan(B, gamma, V, dtype, &P) || V > SV_FILTER_MAX_V) return 0;
  return P.ftotal;
}

int spec_verify_filtered(const void *target_logits, const void *draft_logits, const int32_t *draft_tokens,
                         const float *u_accept, const float *u_sample, const float *temperature,
                         const int32_t *draft_lens, const int32_t *top_k, const float *top_p, int B,
                         int gamma, int V, int dtype, int32_t *accepted_count, int32_t *out_tokens,
                         void *workspace, size_t workspace_bytes, void *stream, const sv_debug *dbg) {
  if (!temperature) return SV_EINVAL;
  return dispatch(target_logits, draft_logits, draft_tokens, u_accept, u_sample, temperature, 0.0f,
                  false, draft_lens, top_k, top_p, B, gamma, V, dtype, accepted_count, out_tokens,
                  workspace, workspace_bytes, stream, dbg);
}

size_t spec_verify_tree_workspace_bytes(int B, int max_nodes, int V, int dtype) {
  Plan P;
  if (max_nodes < 0 || V > SV_TREE_MAX_V || !make_plan(B, max_nodes, V, dtype, &P, SV_TREE_MAX_NODES)) return 0;
  return tree_layout(B, P).total;
}

// Row statistics of every tree position by K1 (the linear layout with
// gamma = max_nodes and draft lengths = node counts; K1 also clears the walk's
// per-request mass words), then NW workgroups per request walk its tree.
int spec_verify_tree(const void *target_logits, const void *draft_logits, const int32_t *node_parent,
                     const int32_t *node_tokens, const int32_t *num_nodes, const float *u_accept,
                     const float *u_sample, const float *temperature, int B, int max_nodes, int V, int dtype,
                     int32_t *accepted_count, int32_t *out_tokens, int32_t *out_nodes, void *workspace,
                     size_t workspace_bytes, void *stream) {
  Plan P;
  if (max_nodes < 0 || V > SV_TREE_MAX_V || !make_plan(B, max_nodes, V, dtype, &P, SV_TREE_MAX_NODES))
    return SV_EINVAL;
  if (P.NS > kTMaxNS) return SV_EINVAL;  // the walk stages a row's chunk partials in LDS
  if (!target_logits || !u_sample || !temperature || !accepted_count || !out_tokens) return SV_EINVAL;
  if (max_nodes > 0 && (!draft_logits || !node_parent || !node_tokens || !u_accept || !out_nodes))
    return SV_EINVAL;
  const TreeLayout L = tree_layout(B, P);
  if (!workspace || (reinterpret_cast<uintptr_t>(workspace) % kAlign) != 0 || workspace_bytes < L.total)
    return SV_EWORKSPACE;
  hipStream_t st = static_cast<hipStream_t>(stream);
  char *base = static_cast<char *>(workspace);
  bool od = max_nodes >= kTreeOnDemandNodes;
  if (const char *m = getenv("SPECVERIFY_TREE_STATS")) {  // a forced choice (testing)
    if (!strcmp(m, "walk")) od = true;
    else if (!strcmp(m, "rows")) od = false;
  }
  if (od) {  // the exchange words (and the error word) start at zero; K1 clears the mass words when it runs
    const long n = static_cast<long>((L.err_off - L.sub_off) / sizeof(unsigned long long)) + 1;
    const long groups = min((n + kBlock - 1) / kBlock, 1024L);
    hipLaunchKernelGGL(k_tree_clear, dim3(static_cast<unsigned>(groups)), dim3(kBlock), 0, st,
                       reinterpret_cast<unsigned long long *>(base + L.sub_off), n);
    if (hipGetLastError() != hipSuccess) return SV_EHIP;
  }
  const int rc = dtype == SV_BF16
                     ? (od ? launch_tree<SV_BF16, true>(target_logits, draft_logits, node_parent, node_tokens,
                                                          num_nodes, u_accept, u_sample, temperature, B, max_nodes,
                                                          V, P, L, base, accepted_count, out_tokens, out_nodes, st)
                           : launch_tree<SV_BF16, false>(target_logits, draft_logits, node_parent, node_tokens,
                                                           num_nodes, u_accept, u_sample, temperature, B, max_nodes,
                                                           V, P, L, base, accepted_count, out_tokens, out_nodes, st))
                     : (od ? launch_tree<SV_F32, true>(target_logits, draft_logits, node_parent, node_tokens,
                                                         num_nodes, u_accept, u_sample, temperature, B, max_nodes, V,
                                                         P, L, base, accepted_count, out_tokens, out_nodes, st)
                           : launch_tree<SV_F32, false>(target_logits, draft_logits, node_parent, node_tokens,
                                                          num_nodes, u_accept, u_sample, temperature, B, max_nodes,
                                                          V, P, L, base, accepted_count, out_tokens, out_nodes, st));
  return rc;
}

size_t spec_sample_workspace_bytes(int R, int V, int dtype) {
  Plan P;
  if (!make_plan(R, 0, V, dtype, &P)) return 0;
  return P.total + align_up(sizeof(int32_t) * static_cast<size_t>(R));
}

// Sampling one token per row: S1 and S2 above (the same law as the verify
// step with no drafts, where every row is a bonus row).
int spec_sample(const void *logits, const float *u, float temperature, const float *temperatures, int R,
                int V, int dtype, int32_t *tokens, void *workspace, size_t workspace_bytes, void *stream) {
  if (!temperatures && (!(temperature >= 0.0f) || isinf(temperature))) return SV_EINVAL;
  Plan P;
  if (!make_plan(R, 0, V, dtype, &P)) return SV_EINVAL;
  if (!logits || !u || !tokens) return SV_EINVAL;
  const size_t need = P.total + align_up(sizeof(int32_t) * static_cast<size_t>(R));
  if (!workspace || (reinterpret_cast<uintptr_t>(workspace) % kAlign) != 0 || workspace_bytes < need)
    return SV_EWORKSPACE;
  // S1 over every row's sub-chunks (records in the workspace's sub-chunk sum
  // area, R * NSUB records of 16 bytes), then S2
  static_assert(sizeof(SubRecord) == sizeof(SubSums), "records share the sub-chunk sum area");
  SubRecord *rec = reinterpret_cast<SubRecord *>(static_cast<char *>(workspace) + P.sums_off);
  const long waves_per_row = min(static_cast<long>(P.NSUB), max(static_cast<long>(kSWaves),
                                                                (kSTargetWaves + R - 1) / R));
  const int SG = static_cast<int>((waves_per_row + kSWaves - 1) / kSWaves);
  if (static_cast<long>(R) * SG > (1L << 32) / kSBlock - 1) return SV_EINVAL;
  hipStream_t st = static_cast<hipStream_t>(stream);
  const dim3 g1(static_cast<unsigned>(static_cast<long>(R) * SG));
  if (dtype == SV_BF16) {
    hipLaunchKernelGGL((k_sample_stats<SV_BF16>), g1, dim3(kSBlock), 0, st, logits, temperatures, temperature, V,
                       P.NSUB, SG, rec);
    hipLaunchKernelGGL((k_sample_pick<SV_BF16>), dim3(R), dim3(kWave), 0, st, logits, u, temperatures,
                       temperature, V, P.NSUB, rec, tokens);
  } else {
    hipLaunchKernelGGL((k_sample_stats<SV_F32>), g1, dim3(kSBlock), 0, st, logits, temperatures, temperature, V,
                       P.NSUB, SG, rec);
    hipLaunchKernelGGL((k_sample_pick<SV_F32>), dim3(R), dim3(kWave), 0, st, logits, u, temperatures,
                       temperature, V, P.NSUB, rec, tokens);
  }
  return hipGetLastError() == hipSuccess ? SV_OK : SV_EHIP;
}

size_t spec_sample_filtered_workspace_bytes(int R, int V, int dtype) {
  Plan P;
  if (!make_plan(R, 0, V, dtype, &P) || V > SV_FILTER_MAX_V) return 0;
  return P.ftotal + align_up(sizeof(int32_t) * static_cast<size_t>(R));
}

// Filtered sampling is the filtered verify step with no drafts: every row is a
// bonus row of its filtered distribution.  The per-row counts (always 0) go to
// the tail of the workspace.
int spec_sample_filtered(const void *logits, const float *u, const float *temperatures, const int32_t *top_k,
                         const float *top_p, int R, int V, int dtype, int32_t *tokens, void *workspace,
                         size_t workspace_bytes, void *stream) {
  Plan P;
  if (!make_plan(R, 0, V, dtype, &P) || V > SV_FILTER_MAX_V) return SV_EINVAL;
  if (!logits || !u || !temperatures || !tokens) return SV_EINVAL;
  const size_t need = P.ftotal + align_up(sizeof(int32_t) * static_cast<size_t>(R));
  if (!workspace || (reinterpret_cast<uintptr_t>(workspace) % kAlign) != 0 || workspace_bytes < need)
    return SV_EWORKSPACE;
  int32_t *counts = reinterpret_cast<int32_t *>(static_cast<char *>(workspace) + P.ftotal);
  return dispatch(logits, nullptr, nullptr, nullptr, u, temperatures, 0.0f, false, nullptr, top_k, top_p, R, 0, V,
                  dtype, counts, tokens, workspace, P.ftotal, stream, nullptr);
}

const char *spec_verify_strerror(int code) {
  switch (code) {
    case SV_OK: return "success";
    case SV_EINVAL: return "invalid argument (pointer, size, dtype or temperature)";
    case SV_EWORKSPACE: return "workspace missing, not 256-byte aligned, or too small";
    case SV_EHIP: return "HIP launch or runtime call failed";
    case SV_ESCRATCH: return "problem too large for the built-in scratch of spec_verify_noalloc";
    default: return "unknown error code";
  }
}

}  // extern "C"
