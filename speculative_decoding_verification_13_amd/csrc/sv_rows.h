// Row and sequence helpers shared by the verification kernels: sequence
// bounds of a ragged batch, the row -> sequence search, the 64-bit chunk
// partials, 16-byte row vectors, and the draw weights of the final inverse CDF.
#pragma once

#include <limits.h>

#include <type_traits>

#include "sv_device.h"
#include "sv_launch.h"

namespace sv {

namespace {

constexpr int kCuLds = 1024;  // offsets staged in LDS for the row -> sequence search

__device__ __forceinline__ bool seq_bounds(const Params& P, int b, int& d0, int& kb) {
  if (P.cu == nullptr) {
    d0 = b * P.K;
    kb = P.K;
    return true;
  }
  const int a = P.cu[b];
  const int e = P.cu[b + 1];
  if (a < 0 || e < a || e > P.total_draft || e - a > SV_MAX_K) return false;
  d0 = a;
  kb = e - a;
  return true;
}

__device__ __forceinline__ bool seq_greedy(const Params& P, int b) {
  return P.all_greedy || (P.greedy != nullptr && P.greedy[b] != 0);
}

// Stats units: draft rows, then target rows (both in row order, so the grid
// streams each logit array linearly).
__device__ __forceinline__ long long unit_of(const Params& P, bool is_target, int row) {
  return is_target ? (long long)P.total_draft + row : (long long)row;
}
__device__ __forceinline__ void row_of_unit(const Params& P, int unit, bool& is_target, int& row) {
  is_target = unit >= P.total_draft;
  row = is_target ? unit - P.total_draft : unit;
}

// (max, sum) of a sampling chunk; NaN is stored canonical. Never all-zero
// bits: a +0 maximum brings a term 2^0 = 1 into the sum.
__device__ __forceinline__ unsigned long long pack_ms(float m, float s) {
  if (m != m) m = __builtin_nanf("");
  return ((unsigned long long)__float_as_uint(s) << 32) | __float_as_uint(m);
}
__device__ __forceinline__ void unpack_ms(unsigned long long v, float& m, float& s) {
  m = __uint_as_float((unsigned)v);
  s = __uint_as_float((unsigned)(v >> 32));
}
// (max value, argmax, bad flag) of a greedy chunk: the high word has bit 31
// set (so the slot is never zero), bit 30 the bad flag, bits 0-29 the argmax
// (an empty chunk's "no index" maps to 2^30 - 1).
__device__ __forceinline__ unsigned long long pack_am(float v, int idx, int bad) {
  const unsigned hi = 0x80000000u | (bad ? 0x40000000u : 0u) | ((unsigned)idx & 0x3fffffffu);
  return ((unsigned long long)hi << 32) | __float_as_uint(v);
}
__device__ __forceinline__ void unpack_am(unsigned long long p, float& v, int& idx, int& bad) {
  v = __uint_as_float((unsigned)p);
  const unsigned hi = (unsigned)(p >> 32);
  idx = (int)(hi & 0x3fffffffu);
  bad = (hi & 0x40000000u) ? 1 : 0;
}
// Merge of a greedy row's C chunk partials, in chunk order (loads issued four
// chunks at a time so their round trips overlap).
__device__ __forceinline__ void merge_greedy(const unsigned long long* tsl, int C, float& v,
                                             int& idx, int& bad) {
  constexpr int G = 4;
  for (int k0 = 0; k0 < C; k0 += G) {
    unsigned long long tv[G];
#pragma unroll
    for (int g = 0; g < G; ++g) tv[g] = (k0 + g < C) ? tsl[k0 + g] : 1ull;
#pragma unroll
    for (int g = 0; g < G; ++g) {
      if (k0 + g < C) {
        float cv;
        int ci, cb;
        unpack_am(tv[g], cv, ci, cb);
        argmax_merge(v, idx, cv, ci);
        bad |= cb;
      }
    }
  }
}

// One 16-byte vector (or one element on the scalar path) of a row.
template <int DT, bool VEC>
struct Vec {
  static constexpr int N = VEC ? Dt<DT>::N : 1;
  using Raw = typename std::conditional<VEC, uint4, float>::type;
  __device__ __forceinline__ static Raw load(const void* base, size_t row_elem, int v) {
    if constexpr (VEC) {
      return reinterpret_cast<const uint4*>(reinterpret_cast<const char*>(base) +
                                            row_elem * Dt<DT>::kBytes)[v];
    } else {
      return load_elem<DT>(base, row_elem + (size_t)v);
    }
  }
  // The same load marked non-temporal (streamed once: not kept in the caches).
  __device__ __forceinline__ static Raw load_stream(const void* base, size_t row_elem, int v) {
    if constexpr (VEC) {
      typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
      const u32x4 t = __builtin_nontemporal_load(
          reinterpret_cast<const u32x4*>(reinterpret_cast<const char*>(base) +
                                         row_elem * Dt<DT>::kBytes) +
          v);
      return make_uint4(t.x, t.y, t.z, t.w);
    } else {
      return load_elem<DT>(base, row_elem + (size_t)v);
    }
  }
  __device__ __forceinline__ static void get(const Raw& r, float* f) {
    if constexpr (VEC) unpack<DT>(r, f);
    else f[0] = r;
  }
};

__device__ __forceinline__ float draw_weight(float lp, float lq, const Job& j, float c) {
  const float ep = (lp >= j.thr_p) ? fast_exp2(fmaf(lp, c, -j.Rp)) : 0.0f;
  if (j.mode == kJobBonus) return ep * j.invSp;
  const float q = (lq >= j.thr_q) ? fast_exp2(fmaf(lq, c, -j.Rq)) * j.invSq : 0.0f;
  return fmaxf(fmaf(ep, j.invSp, -q), 0.0f);
}

// Block reduction of M values per thread; out[u] valid in every thread.
template <int M>
__device__ __forceinline__ void block_sum(const float* v, float* out) {
  __shared__ float s_red[kThreads / kWave][M];
  const int lane = threadIdx.x & (kWave - 1);
  const int w = threadIdx.x / kWave;
  float t[M];
#pragma unroll
  for (int u = 0; u < M; ++u) t[u] = wave_sum(v[u]);
  __syncthreads();
  if (lane == 0) {
#pragma unroll
    for (int u = 0; u < M; ++u) s_red[w][u] = t[u];
  }
  __syncthreads();
#pragma unroll
  for (int u = 0; u < M; ++u) {
    float a = 0.f;
#pragma unroll
    for (int k = 0; k < kThreads / kWave; ++k) a += s_red[k][u];
    out[u] = a;
  }
}
__device__ __forceinline__ void block_sum8(const float* v, float* out) { block_sum<8>(v, out); }

// Sequence of a draft row (is_target false) or target row: the largest b with
// cu[b] <= row, or cu[b] + b <= row. Whole block (stages cu in LDS).
__device__ int row_seq(const Params& P, int row, bool is_target, int* s_cu) {
  if (P.cu == nullptr) return is_target ? row / (P.K + 1) : row / P.K;
  const bool staged = P.B <= kCuLds;
  if (staged) {
    for (int k = threadIdx.x; k < P.B; k += kThreads) s_cu[k] = P.cu[k];
    __syncthreads();
  }
  const int* cu = staged ? s_cu : P.cu;
  int lo = 0, hi = P.B - 1;
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    const long long key = (long long)cu[mid] + (is_target ? mid : 0);
    if (key <= (long long)row) lo = mid;
    else hi = mid - 1;
  }
  return lo;
}

// Whether target row `row` is its sequence's last (bonus) row (whole block).
__device__ __forceinline__ bool is_bonus_row(const Params& P, int row, int* s_cu) {
  if (P.cu == nullptr) return row % (P.K + 1) == P.K;
  const int b = row_seq(P, row, true, s_cu);
  return row == P.cu[b + 1] + b;
}

// Statistics of vectors vb..ve-1 of one row (whole block): for a greedy row
// the argmax (lowest id on ties) and whether the chunk holds NaN or +inf, for a
// sampling row the maximum m and the sum of 2^(l*c - R), R = fp32(m*c).
// Returns the packed partial in thread 0 (0 elsewhere). The loads are streamed
// (non-temporal) unless `stream` is false: rows a draw is likely to read again
// keep the ordinary cache policy. GREEDY_ONLY compiles the greedy statistics
// alone (for callers whose other rows never come here).
template <int DT, bool VEC, bool GREEDY_ONLY = false>
__device__ unsigned long long chunk_stats(const Params& P, const void* base, size_t roff, int vb,
                                          int ve, bool greedy, bool stream = true) {
  using Vc = Vec<DT, VEC>;
  constexpr int N = Vc::N;
  __shared__ float4 s_part[kThreads / kWave];
  const int tid = threadIdx.x;
  const int lane = tid & (kWave - 1);
  const int wave = tid / kWave;
  int v = vb + tid;
  unsigned long long packed;
  if (GREEDY_ONLY || greedy) {
    float bv = kNegInf;
    int bi = INT_MAX, bad = 0;
    for (; v + (kBatch - 1) * kThreads < ve; v += kBatch * kThreads) {
      typename Vc::Raw r[kBatch];
      if (stream) {
#pragma unroll
        for (int u = 0; u < kBatch; ++u) r[u] = Vc::load_stream(base, roff, v + u * kThreads);
      } else {
#pragma unroll
        for (int u = 0; u < kBatch; ++u) r[u] = Vc::load(base, roff, v + u * kThreads);
      }
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int u = 0; u < kBatch; ++u) {
        float f[N];
        Vc::get(r[u], f);
#pragma unroll
        for (int k = 0; k < N; ++k) {
          bad |= is_nan_or_posinf(f[k]);
          if (f[k] > bv) {
            bv = f[k];
            bi = (v + u * kThreads) * N + k;
          }
        }
      }
    }
    for (; v < ve; v += kThreads) {
      float f[N];
      Vc::get(Vc::load_stream(base, roff, v), f);
#pragma unroll
      for (int k = 0; k < N; ++k) {
        bad |= is_nan_or_posinf(f[k]);
        if (f[k] > bv) {
          bv = f[k];
          bi = v * N + k;
        }
      }
    }
    wave_argmax(bv, bi, bad);
    if (lane == 0) s_part[wave] = make_float4(bv, __int_as_float(bi), __int_as_float(bad), 0.f);
    __syncthreads();
    if (tid != 0) return 0ull;
#pragma unroll
    for (int w = 1; w < kThreads / kWave; ++w) {
      argmax_merge(bv, bi, s_part[w].x, __float_as_int(s_part[w].y));
      bad |= __float_as_int(s_part[w].z);
    }
    packed = pack_am(bv, bi, bad);
  } else {
    const float c = P.c;
    float m = kNegInf, s = 0.f;
    for (; v + (kBatch - 1) * kThreads < ve; v += kBatch * kThreads) {
      typename Vc::Raw r[kBatch];
      if (stream) {
#pragma unroll
        for (int u = 0; u < kBatch; ++u) r[u] = Vc::load_stream(base, roff, v + u * kThreads);
      } else {
#pragma unroll
        for (int u = 0; u < kBatch; ++u) r[u] = Vc::load(base, roff, v + u * kThreads);
      }
      __builtin_amdgcn_sched_barrier(0);
      float f[kBatch * N];
#pragma unroll
      for (int u = 0; u < kBatch; ++u) Vc::get(r[u], f + u * N);
      online_update<kBatch * N>(m, s, f, c);
    }
    for (; v < ve; v += kThreads) {
      float f[N];
      Vc::get(Vc::load_stream(base, roff, v), f);
      online_update<N>(m, s, f, c);
    }
    wave_reduce_ms(m, s, c);
    if (lane == 0) s_part[wave] = make_float4(m, s, 0.f, 0.f);
    __syncthreads();
    if (tid != 0) return 0ull;
    // the block's maximum, then every wave's sum at its reference
    float M = s_part[0].x;
#pragma unroll
    for (int w = 1; w < kThreads / kWave; ++w) M = fmaxf(M, s_part[w].x);
    const float RM = ref_of(M, c);
    float S = 0.f;
#pragma unroll
    for (int w = 0; w < kThreads / kWave; ++w) {
      const float sw = s_part[w].y;
      S += (sw == 0.f) ? 0.f : sw * rescale(ref_of(s_part[w].x, c), RM);
    }
    packed = pack_ms(M, S);
  }
  return packed;
}

}  // namespace

}  // namespace sv
