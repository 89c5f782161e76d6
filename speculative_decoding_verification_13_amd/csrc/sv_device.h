// Device-side helpers of the verification kernels (gfx950, wave64).
//
// Numerics: every softmax statistic is kept in base-2 exponent units. For a row
// with raw logits l, temperature T and c = log2(e)/T, the reference of a
// (partial) row is R = fp32(m * c) where m is the raw maximum seen, and the
// partial sum is S = sum 2^(l*c - R) with each exponent formed by one fused
// multiply-add. Every later use of the row (ratio, residual, bonus) forms its
// exponents with the same R and the same fused multiply-add, so the rounding
// of R cancels exactly between numerator and normaliser.
#pragma once

#include <hip/hip_runtime.h>
#include <limits.h>
#include <stdint.h>

#include <type_traits>

#include "spec_verify.h"

namespace sv {

constexpr int kBlock = 256;       // threads of the streaming kernels (4 waves)
constexpr int kWave = 64;
constexpr int kTileElems = 2048;  // residual/bonus tile: one wave, 32 elements/lane
constexpr float kNegInf = -__builtin_huge_valf();
constexpr float kPosInf = __builtin_huge_valf();

template <int DT> struct Dt;
template <> struct Dt<SV_F32> { static constexpr int N = 4; static constexpr int kBytes = 4; };
template <> struct Dt<SV_F16> { static constexpr int N = 8; static constexpr int kBytes = 2; };
template <> struct Dt<SV_BF16> { static constexpr int N = 8; static constexpr int kBytes = 2; };

typedef _Float16 half2_t __attribute__((ext_vector_type(2)));

__device__ __forceinline__ void unpack2(uint32_t w, float& lo, float& hi,
                                        std::integral_constant<int, SV_BF16>) {
  lo = __uint_as_float(w << 16);
  hi = __uint_as_float(w & 0xffff0000u);
}
__device__ __forceinline__ void unpack2(uint32_t w, float& lo, float& hi,
                                        std::integral_constant<int, SV_F16>) {
  half2_t h = __builtin_bit_cast(half2_t, w);
  lo = (float)h.x;
  hi = (float)h.y;
}

// Unpack one 16-byte vector into N floats (exact widening).
template <int DT>
__device__ __forceinline__ void unpack(const uint4 v, float* f) {
  if constexpr (DT == SV_F32) {
    f[0] = __uint_as_float(v.x);
    f[1] = __uint_as_float(v.y);
    f[2] = __uint_as_float(v.z);
    f[3] = __uint_as_float(v.w);
  } else {
    std::integral_constant<int, DT> tag;
    unpack2(v.x, f[0], f[1], tag);
    unpack2(v.y, f[2], f[3], tag);
    unpack2(v.z, f[4], f[5], tag);
    unpack2(v.w, f[6], f[7], tag);
  }
}

// One logit, exact widening. `idx` is an element index from the array base.
template <int DT>
__device__ __forceinline__ float load_elem(const void* base, size_t idx) {
  if constexpr (DT == SV_F32) {
    return reinterpret_cast<const float*>(base)[idx];
  } else {
    uint32_t w = reinterpret_cast<const uint16_t*>(base)[idx];
    if constexpr (DT == SV_BF16) {
      return __uint_as_float(w << 16);
    } else {
      return (float)__builtin_bit_cast(_Float16, (uint16_t)w);
    }
  }
}

// Row reader: VEC = 16-byte vectors (rows 16-byte aligned, V % N == 0), else one
// element per "vector".
template <int DT, bool VEC> struct Reader {
  static constexpr int N = VEC ? Dt<DT>::N : 1;
  // v indexes vectors of the row that starts at element row_elem.
  __device__ __forceinline__ static void load(const void* base, size_t row_elem, int v,
                                              float* f) {
    if constexpr (VEC) {
      const uint4* p = reinterpret_cast<const uint4*>(
          reinterpret_cast<const char*>(base) + row_elem * Dt<DT>::kBytes);
      unpack<DT>(p[v], f);
    } else {
      f[0] = load_elem<DT>(base, row_elem + (size_t)v);
    }
  }
};

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// 2^(a - b) for two references, 1 when equal (covers -inf == -inf).
__device__ __forceinline__ float rescale(float r_old, float r_new) {
  return (r_old == r_new) ? 1.0f : fast_exp2(r_old - r_new);
}

// Reference R = fp32(m * c) of a raw maximum m; 0 for an empty (all -inf) row.
__device__ __forceinline__ float ref_of(float m, float c) {
  return (m == kNegInf) ? 0.0f : m * c;
}

// Merge partial (m, s) statistics: both s are relative to ref_of(their m).
__device__ __forceinline__ void merge_ms(float& m, float& s, float om, float os, float c) {
  const float nm = fmaxf(m, om);
  const float nr = ref_of(nm, c);
  const float a = (s == 0.0f) ? 0.0f : s * rescale(ref_of(m, c), nr);
  const float b = (os == 0.0f) ? 0.0f : os * rescale(ref_of(om, c), nr);
  m = nm;
  s = a + b;
}

// Online update of (m, s) with M values held in registers.
template <int M>
__device__ __forceinline__ void online_update(float& m, float& s, const float* x, float c) {
  float bm = x[0];
#pragma unroll
  for (int k = 1; k < M; ++k) bm = fmaxf(bm, x[k]);
  const float nm = fmaxf(m, bm);
  const float nr = ref_of(nm, c);
  float e[M];
#pragma unroll
  for (int k = 0; k < M; ++k) e[k] = fast_exp2(fmaf(x[k], c, -nr));
#pragma unroll
  for (int w = 1; w < M; w *= 2) {
#pragma unroll
    for (int k = 0; k + w < M; k += 2 * w) e[k] += e[k + w];
  }
  const float old = (s == 0.0f) ? 0.0f : s * rescale(ref_of(m, c), nr);
  s = old + e[0];
  m = nm;
}

// Argmax with lowest index on ties; indices visited in increasing order per
// thread so the strict compare keeps the first maximum.
__device__ __forceinline__ void argmax_merge(float& v, int& i, float ov, int oi) {
  if (ov > v || (ov == v && oi < i)) {
    v = ov;
    i = oi;
  }
}

__device__ __forceinline__ bool is_nan_or_posinf(float x) {
  return __builtin_isfpclass(x, 0x0003 | 0x0200);  // sNaN | qNaN | +inf
}

// ---- wave reductions through DPP (no LDS round trips; every lane active) ----
// Reductions: swap neighbours, swap pairs, mirror half rows, mirror rows (every
// lane of a 16-lane row then holds the row's result), then broadcast lane 15
// into rows 1 and 3 and lane 31 into rows 2 and 3; lane 63 ends with the wave
// result. Inclusive scans: shift right by 1, 2, 4, 8 within each row (lanes
// with no source add the identity), then the same two broadcasts.
template <int CTRL>
__device__ __forceinline__ int dpp_i(int v) {
  return __builtin_amdgcn_mov_dpp(v, CTRL, 0xF, 0xF, false);
}
template <int CTRL, int ROWS>
__device__ __forceinline__ int dpp_rows_i(int v, int ident) {
  return __builtin_amdgcn_update_dpp(ident, v, CTRL, ROWS, 0xF, false);
}
template <int CTRL>
__device__ __forceinline__ float dpp_f(float v) {
  return __builtin_bit_cast(float, dpp_i<CTRL>(__builtin_bit_cast(int, v)));
}
template <int CTRL, int ROWS>
__device__ __forceinline__ float dpp_rows_f(float v, float ident) {
  return __builtin_bit_cast(float, dpp_rows_i<CTRL, ROWS>(__builtin_bit_cast(int, v),
                                                          __builtin_bit_cast(int, ident)));
}
__device__ __forceinline__ float lane63_f(float v) {
  return __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), 63));
}
__device__ __forceinline__ float wave_max_dpp(float v) {
  v = fmaxf(v, dpp_f<0xB1>(v));   // quad_perm [1,0,3,2]
  v = fmaxf(v, dpp_f<0x4E>(v));   // quad_perm [2,3,0,1]
  v = fmaxf(v, dpp_f<0x141>(v));  // row_half_mirror
  v = fmaxf(v, dpp_f<0x140>(v));  // row_mirror
  v = fmaxf(v, dpp_rows_f<0x142, 0xA>(v, kNegInf));  // row_bcast:15
  v = fmaxf(v, dpp_rows_f<0x143, 0xC>(v, kNegInf));  // row_bcast:31
  return lane63_f(v);
}
__device__ __forceinline__ float wave_sum_dpp(float v) {
  v += dpp_f<0xB1>(v);
  v += dpp_f<0x4E>(v);
  v += dpp_f<0x141>(v);
  v += dpp_f<0x140>(v);
  v += dpp_rows_f<0x142, 0xA>(v, 0.0f);
  v += dpp_rows_f<0x143, 0xC>(v, 0.0f);
  return lane63_f(v);
}
__device__ __forceinline__ int wave_min_i(int v) {
  v = min(v, dpp_i<0xB1>(v));
  v = min(v, dpp_i<0x4E>(v));
  v = min(v, dpp_i<0x141>(v));
  v = min(v, dpp_i<0x140>(v));
  v = min(v, dpp_rows_i<0x142, 0xA>(v, INT_MAX));
  v = min(v, dpp_rows_i<0x143, 0xC>(v, INT_MAX));
  return __builtin_amdgcn_readlane(v, 63);
}
__device__ __forceinline__ int wave_max_i(int v) {
  v = max(v, dpp_i<0xB1>(v));
  v = max(v, dpp_i<0x4E>(v));
  v = max(v, dpp_i<0x141>(v));
  v = max(v, dpp_i<0x140>(v));
  v = max(v, dpp_rows_i<0x142, 0xA>(v, INT_MIN));
  v = max(v, dpp_rows_i<0x143, 0xC>(v, INT_MIN));
  return __builtin_amdgcn_readlane(v, 63);
}
__device__ __forceinline__ int wave_sum_i(int v) {
  v += dpp_i<0xB1>(v);
  v += dpp_i<0x4E>(v);
  v += dpp_i<0x141>(v);
  v += dpp_i<0x140>(v);
  v += dpp_rows_i<0x142, 0xA>(v, 0);
  v += dpp_rows_i<0x143, 0xC>(v, 0);
  return __builtin_amdgcn_readlane(v, 63);
}
__device__ __forceinline__ float wave_sum(float x) { return wave_sum_dpp(x); }

__device__ __forceinline__ void wave_merge_ms(float& m, float& s, float c) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) {
    const float om = __shfl_xor(m, o);
    const float os = __shfl_xor(s, o);
    merge_ms(m, s, om, os, c);
  }
}
__device__ __forceinline__ void wave_argmax(float& v, int& i, int& bad) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) {
    const float ov = __shfl_xor(v, o);
    const int oi = __shfl_xor(i, o);
    bad |= __shfl_xor(bad, o);
    argmax_merge(v, i, ov, oi);
  }
}

// Wave-wide (max, sum) of per-lane partials: the maximum first, then each
// lane's sum moved to the maximum's reference (one exponent), then the sum.
__device__ __forceinline__ void wave_reduce_ms(float& m, float& s, float c) {
  const float M = wave_max_dpp(m);
  const float sr = (s == 0.0f) ? 0.0f : s * rescale(ref_of(m, c), ref_of(M, c));
  s = wave_sum_dpp(sr);
  m = M;
}

// Inclusive prefix sum over the wave (lane order).
__device__ __forceinline__ float wave_incl_scan(float x) {
  x += dpp_rows_f<0x111, 0xF>(x, 0.0f);  // row_shr:1
  x += dpp_rows_f<0x112, 0xF>(x, 0.0f);  // row_shr:2
  x += dpp_rows_f<0x114, 0xF>(x, 0.0f);  // row_shr:4
  x += dpp_rows_f<0x118, 0xF>(x, 0.0f);  // row_shr:8
  x += dpp_rows_f<0x142, 0xA>(x, 0.0f);  // row_bcast:15
  x += dpp_rows_f<0x143, 0xC>(x, 0.0f);  // row_bcast:31
  return x;
}

__device__ __forceinline__ int wave_incl_scan_i(int x) {
  x += dpp_rows_i<0x111, 0xF>(x, 0);  // row_shr:1
  x += dpp_rows_i<0x112, 0xF>(x, 0);  // row_shr:2
  x += dpp_rows_i<0x114, 0xF>(x, 0);  // row_shr:4
  x += dpp_rows_i<0x118, 0xF>(x, 0);  // row_shr:8
  x += dpp_rows_i<0x142, 0xA>(x, 0);  // row_bcast:15
  x += dpp_rows_i<0x143, 0xC>(x, 0);  // row_bcast:31
  return x;
}

// Bitonic sort of one (value, weight) pair per lane across the wave, by value
// in descending order (lane 0 ends with the largest). Each compare-exchange
// keeps its own pair on equal values, so pairs are permuted, never copied.
__device__ __forceinline__ void wave_sort_desc(float& v, float& w) {
  const int lane = threadIdx.x & (kWave - 1);
#pragma unroll
  for (int size = 2; size <= kWave; size <<= 1) {
#pragma unroll
    for (int stride = size >> 1; stride > 0; stride >>= 1) {
      const float ov = __shfl_xor(v, stride);
      const float ow = __shfl_xor(w, stride);
      // descending runs where (lane & size) == 0, ascending elsewhere; the
      // lower lane of a pair takes the larger value in a descending run
      const bool keep_max = ((lane & size) == 0) == ((lane & stride) == 0);
      if (keep_max ? (ov > v) : (ov < v)) {
        v = ov;
        w = ow;
      }
    }
  }
}

// Bitonic sort of one (id, two payloads) triple per lane across the wave, by
// id in ascending order (ids distinct, or pads of INT_MAX that sort last).
__device__ __forceinline__ void wave_sort_by_id(int& id, float& a, float& b) {
  const int lane = threadIdx.x & (kWave - 1);
#pragma unroll
  for (int size = 2; size <= kWave; size <<= 1) {
#pragma unroll
    for (int stride = size >> 1; stride > 0; stride >>= 1) {
      const int oid = __shfl_xor(id, stride);
      const float oa = __shfl_xor(a, stride);
      const float ob = __shfl_xor(b, stride);
      // ascending runs where (lane & size) == 0; the lower lane of a pair
      // takes the smaller id in an ascending run
      const bool keep_min = ((lane & size) == 0) == ((lane & stride) == 0);
      if (keep_min ? (oid < id) : (oid > id)) {
        id = oid;
        a = oa;
        b = ob;
      }
    }
  }
}

// Block-wide inclusive scan for kBlock threads; `total` receives the block sum.
__device__ __forceinline__ float block_incl_scan(float x, float& total) {
  __shared__ float s_w[kBlock / kWave];
  const int lane = threadIdx.x & (kWave - 1);
  const int w = threadIdx.x / kWave;
  float incl = wave_incl_scan(x);
  __syncthreads();
  if (lane == kWave - 1) s_w[w] = incl;
  __syncthreads();
  float base = 0.0f;
  total = 0.0f;
#pragma unroll
  for (int k = 0; k < kBlock / kWave; ++k) {
    const float t = s_w[k];
    if (k < w) base += t;
    total += t;
  }
  return base + incl;
}

__device__ __forceinline__ int block_min_i(int x) {
  __shared__ int s_w[kBlock / kWave];
  x = wave_min_i(x);
  __syncthreads();
  if ((threadIdx.x & (kWave - 1)) == 0) s_w[threadIdx.x / kWave] = x;
  __syncthreads();
  int r = s_w[0];
#pragma unroll
  for (int k = 1; k < kBlock / kWave; ++k) r = min(r, s_w[k]);
  return r;
}
__device__ __forceinline__ int block_max_i(int x) {
  __shared__ int s_w[kBlock / kWave];
  x = wave_max_i(x);
  __syncthreads();
  if ((threadIdx.x & (kWave - 1)) == 0) s_w[threadIdx.x / kWave] = x;
  __syncthreads();
  int r = s_w[0];
#pragma unroll
  for (int k = 1; k < kBlock / kWave; ++k) r = max(r, s_w[k]);
  return r;
}

// Smallest thread index of the block whose `pred` holds (INT_MAX if none), and
// the largest (-1 if none), through one ballot per wave.
__device__ __forceinline__ int block_first_lane(bool pred) {
  __shared__ int s_w[kBlock / kWave];
  const unsigned long long m = __ballot(pred);
  __syncthreads();
  if ((threadIdx.x & (kWave - 1)) == 0)
    s_w[threadIdx.x / kWave] = m ? (int)(threadIdx.x + __ffsll((long long)m) - 1) : INT_MAX;
  __syncthreads();
  int r = s_w[0];
#pragma unroll
  for (int k = 1; k < kBlock / kWave; ++k) r = min(r, s_w[k]);
  return r;
}
__device__ __forceinline__ int block_last_lane(bool pred) {
  __shared__ int s_w[kBlock / kWave];
  const unsigned long long m = __ballot(pred);
  __syncthreads();
  if ((threadIdx.x & (kWave - 1)) == 0)
    s_w[threadIdx.x / kWave] = m ? (int)(threadIdx.x + 63 - __clzll((long long)m)) : -1;
  __syncthreads();
  int r = s_w[0];
#pragma unroll
  for (int k = 1; k < kBlock / kWave; ++k) r = max(r, s_w[k]);
  return r;
}

// Block-wide exclusive scan of ints for kBlock threads; `total` receives the sum.
__device__ __forceinline__ int block_excl_scan_i(int x, int& total) {
  __shared__ int s_w[kBlock / kWave];
  const int lane = threadIdx.x & (kWave - 1);
  const int w = threadIdx.x / kWave;
  const int incl = wave_incl_scan_i(x);
  __syncthreads();
  if (lane == kWave - 1) s_w[w] = incl;
  __syncthreads();
  int base = 0;
  total = 0;
#pragma unroll
  for (int k = 0; k < kBlock / kWave; ++k) {
    const int t = s_w[k];
    if (k < w) base += t;
    total += t;
  }
  return base + incl - x;
}

__device__ __forceinline__ float block_max_f(float x) {
  __shared__ float s_w[kBlock / kWave];
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) x = fmaxf(x, __shfl_xor(x, o));
  __syncthreads();
  if ((threadIdx.x & (kWave - 1)) == 0) s_w[threadIdx.x / kWave] = x;
  __syncthreads();
  float r = s_w[0];
#pragma unroll
  for (int k = 1; k < kBlock / kWave; ++k) r = fmaxf(r, s_w[k]);
  return r;
}

__device__ __forceinline__ int block_sum_i(int x) {
  __shared__ int s_w[kBlock / kWave];
  x = wave_sum_i(x);
  __syncthreads();
  if ((threadIdx.x & (kWave - 1)) == 0) s_w[threadIdx.x / kWave] = x;
  __syncthreads();
  int r = 0;
#pragma unroll
  for (int k = 0; k < kBlock / kWave; ++k) r += s_w[k];
  return r;
}

// Radix-select step over a histogram of BINS bins (whole block; wave 0 works):
// the largest bin b with (count of bins above b) < rem <= (count of bins >= b),
// written as s_sel[0] = b and s_sel[1] = rem - (count of bins above b). Lane
// l first sums the BINS/64 bins below BINS - 1 - l*BINS/64 (lane 0 holds the
// top); a scan over the lanes finds the lane whose bins hold the rank, and a
// second scan over that lane's bins, one per lane, finds the bin. If rem
// exceeds every count (not reachable for a valid rank) the lowest bin is taken.
template <int BINS = 256>
__device__ __forceinline__ void select_bin(const int* s_hist, int rem, int* s_sel) {
  constexpr int PER = BINS / kWave;
  static_assert(PER * kWave == BINS && PER <= kWave, "bins must fill the wave's lanes evenly");
  if (threadIdx.x < kWave) {
    const int lane = threadIdx.x;
    const int top = BINS - 1 - PER * lane;
    int sum = 0;
#pragma unroll
    for (int j = 0; j < PER; ++j) sum += s_hist[top - j];
    const int incl = wave_incl_scan_i(sum);
    const unsigned long long hit = __ballot(incl >= rem);
    const int first = hit ? (__ffsll(hit) - 1) : (kWave - 1);
    const int above = __shfl(incl - sum, first);  // count of the bins above lane first's
    const int ftop = BINS - 1 - PER * first;
    const int c = lane < PER ? s_hist[ftop - lane] : 0;
    const int ci = wave_incl_scan_i(c);
    const unsigned long long hit2 = __ballot(lane < PER && above + ci >= rem);
    const int j = hit2 ? (__ffsll(hit2) - 1) : (PER - 1);
    if (lane == j) {
      s_sel[0] = ftop - j;
      s_sel[1] = rem - (above + ci - c);
    }
  }
}

// Order-preserving 32-bit key of a non-NaN float (-0 and +0 share one key).
__device__ __forceinline__ unsigned key_of(float f) {
  const unsigned u = __float_as_uint(f == 0.0f ? 0.0f : f);
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}
__device__ __forceinline__ float float_of_key(unsigned k) {
  return __uint_as_float((k & 0x80000000u) ? (k & 0x7fffffffu) : ~k);
}

// ---- cross-block publication (agent scope, no L2 writeback/invalidate) ----
// Shared records are written with agent-scope atomic stores, which write
// through to the device coherence point, and read with agent-scope atomic
// loads. A writer drains its stores (vmcnt) before it bumps a counter, so a
// reader that has seen the counter reads the published values.
__device__ __forceinline__ void pub_f(float* p, float v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void pub_i(int* p, int v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void pub_u64(unsigned long long* p, unsigned long long v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ unsigned long long obs_u64(const unsigned long long* p) {
  return __hip_atomic_load(const_cast<unsigned long long*>(p), __ATOMIC_RELAXED,
                           __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ float obs_f(const float* p) {
  return __hip_atomic_load(const_cast<float*>(p), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ int obs_i(const int* p) {
  return __hip_atomic_load(const_cast<int*>(p), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void drain_stores() { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); }
__device__ __forceinline__ void compiler_fence() { asm volatile("" ::: "memory"); }
__device__ __forceinline__ int bump(int* p, int v = 1) {
  return __hip_atomic_fetch_add(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void raise_flag(int* p, int bits) {
  __hip_atomic_fetch_or(p, bits, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

}  // namespace sv
