// HIP kernels of the batched speculative-decoding verification step (gfx950).
//
// A call runs four kernels on the caller's stream:
//   1. k_row_stats   grid (target row, V-chunk): streams the draft and target
//                    row chunk once with 16-byte loads and keeps an online
//                    (max, sum 2^(l*c - R)) per row; greedy sequences keep an
//                    argmax of the target row instead and skip the draft row.
//   2. k_decide      one wave per sequence: merges the chunk partials, forms
//                    r_i = p_i(x_i)/q_i(x_i), tests u_i < r_i on each lane,
//                    finds the first rejection with a ballot, writes the
//                    accepted prefix and the job of the final draw.
//   3. k_resid_tiles grid (sequence, tile group): per 2048-element tile the sum
//                    of the final draw's weights: max(0, p_n - q_n) after a
//                    rejection, p_K for the bonus.
//   4. k_resid_pick  one block per sequence: scans the tile sums, finds the tile
//                    holding u*Z, scans inside it and writes the token.
// Pages (by title, section): aivaro.ru answer 289 "Как работает speculative
// decoding на уровне логитов, а не токенов?" s.5 step 3, s.6, s.9; Hung-yi Lee
// lecture-16 notes part "4、推测解码验证流程图" items 1-4; aihero.vn
// "Speculative decoding" section "Chấp nhận bằng tỉ lệ, không chỉ bằng argmax".
#include <limits.h>

#include "sv_device.h"
#include "sv_launch.h"

namespace sv {

namespace {

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

// Sequence owning target row g: the largest b with cu[b] + b <= g.
__device__ __forceinline__ int seq_of_target_row(const Params& P, int g) {
  if (P.cu == nullptr) return g / (P.K + 1);
  int lo = 0, hi = P.B - 1;
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if ((long long)P.cu[mid] + mid <= (long long)g) lo = mid;
    else hi = mid - 1;
  }
  return lo;
}

__device__ __forceinline__ bool seq_greedy(const Params& P, int b) {
  return P.all_greedy || (P.greedy != nullptr && P.greedy[b] != 0);
}

}  // namespace

// ---------------------------------------------------------------------------
// 1. Row statistics over one V-chunk of one (draft row, target row) pair.
// ---------------------------------------------------------------------------
template <int DT, bool VEC>
__global__ __launch_bounds__(kBlock) void k_row_stats(const Params P) {
  using Rd = Reader<DT, VEC>;
  constexpr int N = Rd::N;
  constexpr int U = VEC ? 4 : 8;  // vectors of each row in flight per thread
  const int g = blockIdx.x / P.chunks;
  const int ch = blockIdx.x - g * P.chunks;
  const int b = seq_of_target_row(P, g);
  int d0, kb;
  if (!seq_bounds(P, b, d0, kb)) return;
  const int i = g - (d0 + b);
  if (i < 0 || i > kb) return;
  const bool greedy = seq_greedy(P, b);
  const int vbeg = ch * P.chunk_vecs;
  const int vend = min(P.nvec, vbeg + P.chunk_vecs);
  const size_t prow = (size_t)g * (size_t)P.V;
  const int tid = threadIdx.x;
  const int lane = tid & (kWave - 1);
  const int wave = tid / kWave;
  __shared__ float4 s_part[kBlock / kWave];
  float4 rec;

  if (greedy) {
    float bv = kNegInf;
    int bi = INT_MAX;
    int bad = 0;
    int v = vbeg + tid;
    for (; v + (U - 1) * kBlock < vend; v += U * kBlock) {
      float f[U][N];
#pragma unroll
      for (int u = 0; u < U; ++u) Rd::load(P.target, prow, v + u * kBlock, f[u]);
#pragma unroll
      for (int u = 0; u < U; ++u)
#pragma unroll
        for (int k = 0; k < N; ++k) {
          const float x = f[u][k];
          bad |= is_nan_or_posinf(x);
          if (x > bv) {
            bv = x;
            bi = (v + u * kBlock) * N + k;
          }
        }
    }
    for (; v < vend; v += kBlock) {
      float f[N];
      Rd::load(P.target, prow, v, f);
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
    if (tid == 0) {
#pragma unroll
      for (int w = 1; w < kBlock / kWave; ++w) {
        argmax_merge(bv, bi, s_part[w].x, __float_as_int(s_part[w].y));
        bad |= __float_as_int(s_part[w].z);
      }
      rec = make_float4(bv, __int_as_float(bi), __int_as_float(bad), 0.f);
    }
  } else {
    const float c = P.c;
    const bool has_draft = i < kb;
    const size_t qrow = (size_t)(d0 + i) * (size_t)P.V;
    float mq = kNegInf, sq = 0.f, mp = kNegInf, sp = 0.f;
    int v = vbeg + tid;
    if (has_draft) {
      for (; v + (U - 1) * kBlock < vend; v += U * kBlock) {
        float fp[U * N], fq[U * N];
#pragma unroll
        for (int u = 0; u < U; ++u) {
          Rd::load(P.target, prow, v + u * kBlock, fp + u * N);
          Rd::load(P.draft, qrow, v + u * kBlock, fq + u * N);
        }
        online_update<U * N>(mp, sp, fp, c);
        online_update<U * N>(mq, sq, fq, c);
      }
      for (; v < vend; v += kBlock) {
        float fp[N], fq[N];
        Rd::load(P.target, prow, v, fp);
        Rd::load(P.draft, qrow, v, fq);
        online_update<N>(mp, sp, fp, c);
        online_update<N>(mq, sq, fq, c);
      }
    } else {
      for (; v + (U - 1) * kBlock < vend; v += U * kBlock) {
        float fp[U * N];
#pragma unroll
        for (int u = 0; u < U; ++u) Rd::load(P.target, prow, v + u * kBlock, fp + u * N);
        online_update<U * N>(mp, sp, fp, c);
      }
      for (; v < vend; v += kBlock) {
        float fp[N];
        Rd::load(P.target, prow, v, fp);
        online_update<N>(mp, sp, fp, c);
      }
    }
    wave_merge_ms(mq, sq, c);
    wave_merge_ms(mp, sp, c);
    if (lane == 0) s_part[wave] = make_float4(mq, sq, mp, sp);
    __syncthreads();
    if (tid == 0) {
#pragma unroll
      for (int w = 1; w < kBlock / kWave; ++w) {
        merge_ms(mq, sq, s_part[w].x, s_part[w].y, c);
        merge_ms(mp, sp, s_part[w].z, s_part[w].w, c);
      }
      rec = make_float4(mq, sq, mp, sp);
    }
  }
  if (tid == 0) P.partials[(size_t)g * P.chunks + ch] = rec;
}

// ---------------------------------------------------------------------------
// 2. Per-sequence decision: one thread per position i in [0, K_b] (K_b <= 64,
// so 65 positions: two waves). Draft positions all sit in wave 0, whose ballot
// gives the first rejection.
// ---------------------------------------------------------------------------
constexpr int kDecideThreads = 2 * kWave;

template <int DT>
__global__ __launch_bounds__(kDecideThreads) void k_decide(const Params P) {
  __shared__ float s_m[2][SV_MAX_K + 1];
  __shared__ float s_s[2][SV_MAX_K + 1];
  __shared__ int s_gi[SV_MAX_K + 1];
  __shared__ int s_flags;
  __shared__ unsigned long long s_rej;
  const int b = blockIdx.x;
  const int tid = threadIdx.x;
  int d0, kb;
  if (!seq_bounds(P, b, d0, kb)) {
    if (tid == 0) {
      P.num_accepted[b] = SV_SEQ_BAD_OFFSETS;
      P.jobs[b].mode = kJobNone;
    }
    return;
  }
  if (tid == 0) {
    s_flags = 0;
    s_rej = 0ull;
  }
  __syncthreads();
  const float c = P.c;
  const int t0 = d0 + b;
  const bool greedy = seq_greedy(P, b);
  const bool active = tid <= kb;
  const bool is_draft = tid < kb;

  float mq = kNegInf, sq = 0.f, mp = kNegInf, sp = 0.f;
  float gv = kNegInf;
  int gi = INT_MAX, gbad = 0;
  if (active) {
    const float4* rp = P.partials + (size_t)(t0 + tid) * P.chunks;
    for (int k = 0; k < P.chunks; ++k) {
      const float4 r = rp[k];
      if (greedy) {
        argmax_merge(gv, gi, r.x, __float_as_int(r.y));
        gbad |= __float_as_int(r.z);
      } else {
        merge_ms(mq, sq, r.x, r.y, c);
        merge_ms(mp, sp, r.z, r.w, c);
      }
    }
    s_m[0][tid] = mq;
    s_s[0][tid] = sq;
    s_m[1][tid] = mp;
    s_s[1][tid] = sp;
    s_gi[tid] = gi;
  }
  bool row_ok = true;
  if (active) {
    if (greedy) {
      row_ok = !gbad && gv != kNegInf;
    } else {
      row_ok = __builtin_isfinite(mp) && sp > 0.f && __builtin_isfinite(sp);
      if (is_draft) row_ok = row_ok && __builtin_isfinite(mq) && sq > 0.f && __builtin_isfinite(sq);
    }
  }
  int x = -1;
  bool tok_ok = true;
  if (is_draft) {
    x = P.tokens[d0 + tid];
    tok_ok = x >= 0 && x < P.V;
  }
  bool acc = true;
  float ratio = __builtin_nanf("");
  if (is_draft && tok_ok && row_ok) {
    if (greedy) {
      acc = (gi == x);
    } else {
      // r = p(x)/q(x) = 2^((lp*c - Rp) - (lq*c - Rq)) * Sq / Sp
      const float lq = load_elem<DT>(P.draft, (size_t)(d0 + tid) * P.V + x);
      const float lp = load_elem<DT>(P.target, (size_t)(t0 + tid) * P.V + x);
      const float ep = fmaf(lp, c, -ref_of(mp, c));
      const float eq = fmaf(lq, c, -ref_of(mq, c));
      ratio = fast_exp2(ep - eq) * (sq / sp);
      acc = P.uniforms[t0 + tid] < ratio;  // strict: u == r rejects
    }
  }
  if (active && !row_ok) atomicOr(&s_flags, 2);
  if (is_draft && !tok_ok) atomicOr(&s_flags, 1);
  if (tid < kWave) {
    const unsigned long long rej = __ballot(is_draft && !acc);
    if (tid == 0) s_rej = rej;
  }
  __syncthreads();
  const int flags = s_flags;
  const unsigned long long rej = s_rej;
  const int code = (flags & 1) ? SV_SEQ_BAD_TOKEN : ((flags & 2) ? SV_SEQ_BAD_ROW : 0);
  const int n = rej ? (__ffsll(rej) - 1) : kb;

  if (active) {
    int tok = -1;
    if (code == 0) {
      if (tid < n) tok = x;
      else if (tid == n && greedy) tok = gi;
    }
    P.out_tokens[t0 + tid] = tok;
  }
  if (tid == 0) {
    P.num_accepted[b] = code ? code : n;
    Job j;
    j.mode = (code != 0 || greedy) ? kJobNone : (n < kb ? kJobResidual : kJobBonus);
    j.n = n;
    j.qrow = d0 + n;
    j.prow = t0 + n;
    j.out_idx = t0 + n;
    j.Rq = ref_of(s_m[0][n], c);
    j.invSq = 1.0f / s_s[0][n];
    j.Rp = ref_of(s_m[1][n], c);
    j.invSp = 1.0f / s_s[1][n];
    j.u = (j.mode != kJobNone) ? P.uniforms[t0 + kb] : 0.f;
    P.jobs[b] = j;
  }
  // side outputs
  const float kLn2 = 0.69314718055994531f;
  const float nan = __builtin_nanf("");
  if (active && P.diag.row_max_target) P.diag.row_max_target[t0 + tid] = greedy ? gv : mp;
  if (active && P.diag.row_logsum_target)
    P.diag.row_logsum_target[t0 + tid] =
        greedy ? nan : (__log2f(sp) + fmaf(-mp, c, ref_of(mp, c))) * kLn2;
  if (is_draft && P.diag.row_max_draft) P.diag.row_max_draft[d0 + tid] = greedy ? nan : mq;
  if (is_draft && P.diag.row_logsum_draft)
    P.diag.row_logsum_draft[d0 + tid] =
        greedy ? nan : (__log2f(sq) + fmaf(-mq, c, ref_of(mq, c))) * kLn2;
  if (is_draft && P.diag.ratio) P.diag.ratio[d0 + tid] = ratio;
  if (tid == 0 && P.diag.resid_Z && (code != 0 || greedy)) P.diag.resid_Z[b] = nan;
}

// ---------------------------------------------------------------------------
// 3./4. Final draw: weights w(x) of the residual (after a rejection) or of the
// bonus row; inverse CDF over ascending ids.
// ---------------------------------------------------------------------------
template <int DT>
__device__ __forceinline__ float draw_weight(float lp, float lq, int mode, const Job& j, float c) {
  const float ep = fast_exp2(fmaf(lp, c, -j.Rp));
  if (mode == kJobBonus) return ep * j.invSp;
  const float q = fast_exp2(fmaf(lq, c, -j.Rq)) * j.invSq;
  return fmaxf(fmaf(ep, j.invSp, -q), 0.0f);
}

// Sum of this lane's share of tile t's weights (one wave covers the tile).
template <int DT, bool VEC>
__device__ __forceinline__ float tile_lane_sum(const Params& P, const Job& j, int mode, int t,
                                               int lane) {
  const size_t prow = (size_t)j.prow * P.V;
  const size_t qrow = (size_t)j.qrow * P.V;
  float acc = 0.f;
  if constexpr (VEC) {
    using Rd = Reader<DT, true>;
    constexpr int N = Rd::N;
    constexpr int KV = kTileElems / (kWave * N);  // vectors per lane
    const int vb = t * (kTileElems / N);
#pragma unroll
    for (int k = 0; k < KV; ++k) {
      const int v = vb + k * kWave + lane;
      if (v < P.nvec) {
        float fp[N], fq[N];
        Rd::load(P.target, prow, v, fp);
        if (mode == kJobResidual) Rd::load(P.draft, qrow, v, fq);
        float s = 0.f;
#pragma unroll
        for (int e = 0; e < N; ++e) s += draw_weight<DT>(fp[e], fq[e], mode, j, P.c);
        acc += s;
      }
    }
  } else {
    const int eb = t * kTileElems;
    for (int k = 0; k < kTileElems / kWave; ++k) {
      const int e = eb + k * kWave + lane;
      if (e < P.V) {
        const float lp = load_elem<DT>(P.target, prow + e);
        const float lq = (mode == kJobResidual) ? load_elem<DT>(P.draft, qrow + e) : 0.f;
        acc += draw_weight<DT>(lp, lq, mode, j, P.c);
      }
    }
  }
  return acc;
}

template <int DT, bool VEC>
__global__ __launch_bounds__(kBlock) void k_resid_tiles(const Params P) {
  const int b = blockIdx.x / P.tile_chunks;
  const int ch = blockIdx.x - b * P.tile_chunks;
  const Job j = P.jobs[b];
  if (j.mode == kJobNone) return;
  const int lane = threadIdx.x & (kWave - 1);
  const int wave = threadIdx.x / kWave;
  const int t_beg = ch * P.tiles_per_chunk;
  const int t_end = min(P.ntiles, t_beg + P.tiles_per_chunk);
  for (int t = t_beg + wave; t < t_end; t += kBlock / kWave) {
    const float s = wave_sum(tile_lane_sum<DT, VEC>(P, j, j.mode, t, lane));
    if (lane == 0) P.tile_sums[(size_t)b * P.ntiles + t] = s;
  }
}

// Finds the first tile whose inclusive prefix exceeds u*Z (or the last tile with
// positive mass). Returns the tile; sets Z and the exclusive prefix `base`.
__device__ __forceinline__ int find_tile(const float* ts, int ntiles, float u, float& Z,
                                         float& target, float& base) {
  __shared__ float s_base;
  const int per = (ntiles + kBlock - 1) / kBlock;
  const int t0 = threadIdx.x * per;
  const int t1 = min(ntiles, t0 + per);
  float local = 0.f;
  for (int t = t0; t < t1; ++t) local += ts[t];
  float total;
  const float incl = block_incl_scan(local, total);
  Z = total;
  target = u * total;
  float run = incl - local;
  int cand = INT_MAX, lastpos = -1;
  for (int t = t0; t < t1; ++t) {
    const float w = ts[t];
    const float nxt = run + w;
    if (cand == INT_MAX && nxt > target) cand = t;
    if (w > 0.f) lastpos = t;
    run = nxt;
  }
  int tile = block_min_i(cand);
  if (tile == INT_MAX) tile = block_max_i(lastpos);
  if (tile < 0) tile = 0;
  // exclusive prefix of the chosen tile, from its owner thread
  __syncthreads();
  if (tile >= t0 && tile < t1) {
    float r = incl - local;
    for (int t = t0; t < tile; ++t) r += ts[t];
    s_base = r;
  }
  __syncthreads();
  base = s_base;
  return tile;
}

template <int DT, bool VEC>
__global__ __launch_bounds__(kBlock) void k_resid_pick(const Params P) {
  const int b = blockIdx.x;
  const Job j = P.jobs[b];
  if (j.mode == kJobNone) return;
  float* ts = P.tile_sums + (size_t)b * P.ntiles;
  int mode = j.mode;
  float Z, target, base;
  int tile = find_tile(ts, P.ntiles, j.u, Z, target, base);
  if (!(Z > 0.f) && mode == kJobResidual) {
    // Residual mass rounded to zero: draw from p_n instead.
    mode = kJobBonus;
    const int lane = threadIdx.x & (kWave - 1);
    const int wave = threadIdx.x / kWave;
    __syncthreads();
    for (int t = wave; t < P.ntiles; t += kBlock / kWave) {
      const float s = wave_sum(tile_lane_sum<DT, VEC>(P, j, mode, t, lane));
      if (lane == 0) ts[t] = s;
    }
    __threadfence_block();
    __syncthreads();
    tile = find_tile(ts, P.ntiles, j.u, Z, target, base);
  }
  // In-tile scan: thread t owns 8 consecutive ids of the tile.
  constexpr int E = kTileElems / kBlock;
  const int e0 = tile * kTileElems + threadIdx.x * E;
  const size_t prow = (size_t)j.prow * P.V;
  const size_t qrow = (size_t)j.qrow * P.V;
  float w[E];
  float run = 0.f;
#pragma unroll
  for (int k = 0; k < E; ++k) {
    const int e = e0 + k;
    float wk = 0.f;
    if (e < P.V) {
      const float lp = load_elem<DT>(P.target, prow + e);
      const float lq = (mode == kJobResidual) ? load_elem<DT>(P.draft, qrow + e) : 0.f;
      wk = draw_weight<DT>(lp, lq, mode, j, P.c);
    }
    run += wk;
    w[k] = run;  // local inclusive prefix
  }
  float tot;
  const float incl = block_incl_scan(run, tot);
  const float excl = base + (incl - run);
  int cand = INT_MAX, lastpos = -1;
  float prev = 0.f;
#pragma unroll
  for (int k = 0; k < E; ++k) {
    if (cand == INT_MAX && excl + w[k] > target) cand = e0 + k;
    if (w[k] > prev) lastpos = e0 + k;
    prev = w[k];
  }
  int tok = block_min_i(cand);
  if (tok == INT_MAX) tok = block_max_i(lastpos);
  if (tok < 0) tok = tile * kTileElems;
  if (threadIdx.x == 0) {
    P.out_tokens[j.out_idx] = tok;
    if (P.diag.resid_Z) P.diag.resid_Z[b] = Z;
  }
}

__global__ void k_fill_zero(uint4* p, size_t n16) {
  for (size_t k = (size_t)blockIdx.x * blockDim.x + threadIdx.x; k < n16;
       k += (size_t)gridDim.x * blockDim.x)
    p[k] = make_uint4(0, 0, 0, 0);
}

// ---------------------------------------------------------------------------
// Host side: launch sequence.
// ---------------------------------------------------------------------------
template <int DT, bool VEC>
static hipError_t launch_all(const Params& P, const Plan& L, hipStream_t s, hipEvent_t* ev,
                             int nev) {
  int e = 0;
  auto mark = [&]() -> hipError_t {
    if (ev != nullptr && e < nev) return hipEventRecord(ev[e++], s);
    return hipSuccess;
  };
  hipError_t err;
  if ((err = mark()) != hipSuccess) return err;
  hipLaunchKernelGGL((k_row_stats<DT, VEC>), dim3(L.stats_blocks), dim3(kBlock), 0, s, P);
  if ((err = hipGetLastError()) != hipSuccess || (err = mark()) != hipSuccess) return err;
  hipLaunchKernelGGL((k_decide<DT>), dim3(P.B), dim3(kDecideThreads), 0, s, P);
  if ((err = hipGetLastError()) != hipSuccess || (err = mark()) != hipSuccess) return err;
  if (!L.any_sampling) return hipSuccess;
  hipLaunchKernelGGL((k_resid_tiles<DT, VEC>), dim3(L.tile_blocks), dim3(kBlock), 0, s, P);
  if ((err = hipGetLastError()) != hipSuccess || (err = mark()) != hipSuccess) return err;
  hipLaunchKernelGGL((k_resid_pick<DT, VEC>), dim3(P.B), dim3(kBlock), 0, s, P);
  if ((err = hipGetLastError()) != hipSuccess || (err = mark()) != hipSuccess) return err;
  return hipSuccess;
}

hipError_t launch(int dtype, bool vec, const Params& P, const Plan& L, hipStream_t s,
                  hipEvent_t* ev, int nev) {
  switch (dtype) {
    case SV_F32:
      return vec ? launch_all<SV_F32, true>(P, L, s, ev, nev)
                 : launch_all<SV_F32, false>(P, L, s, ev, nev);
    case SV_F16:
      return vec ? launch_all<SV_F16, true>(P, L, s, ev, nev)
                 : launch_all<SV_F16, false>(P, L, s, ev, nev);
    default:
      return vec ? launch_all<SV_BF16, true>(P, L, s, ev, nev)
                 : launch_all<SV_BF16, false>(P, L, s, ev, nev);
  }
}

hipError_t fill_zero(void* p, size_t bytes, hipStream_t s) {
  const size_t n16 = bytes / 16;
  if (n16 == 0) return hipSuccess;
  const unsigned blocks = (unsigned)((n16 + 255) / 256 < 1024 ? (n16 + 255) / 256 : 1024);
  hipLaunchKernelGGL(k_fill_zero, dim3(blocks), dim3(256), 0, s, reinterpret_cast<uint4*>(p), n16);
  return hipGetLastError();
}

}  // namespace sv
