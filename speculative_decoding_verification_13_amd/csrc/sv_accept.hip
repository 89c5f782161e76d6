// Acceptance statistics of sampling verification for gfx950: for every draft
// position the probability that a draft drawn from q passes the ratio test,
//   beta = sum_x q(x) * min(1, p(x)/q(x)) = sum_x min(p(x), q(x)),
// and for every sequence the expected number of accepted drafts of a round,
//   E[n] = sum_{j<K_b} prod_{i<=j} beta_i
// (the walk stops at the first rejection; the rows are held fixed).
//
// Two passes over the rows: the statistics pass (sv_verify.hip: chunk
// partials, and with top-k the per-row filter) gives each row's maximum, sum
// and kept-set threshold; k_beta then streams both rows of every pair again.
// Block (pair, chunk) merges the pair's row partials in chunk order (every
// block of the pair gets the same values), sums min(p, q) over its chunk and
// publishes the sum; the last block of the pair to finish adds the chunk sums
// in chunk order, writes beta and returns the pair's partials and counter to
// zero. k_expect forms E[n] per sequence.
//
// Pages (by title, section): aivaro.ru answer 289 "Как работает speculative
// decoding на уровне логитов, а не токенов?" s.6 (a draft token passes with
// probability min(1, p/q); the acceptance rate measures how close the draft
// is to the target); aihero.vn "Speculative decoding" section "Khi thời gian
// tiết kiệm bị chi phí ăn hết" (measure useful tokens per round and the
// acceptance rate); Hung-yi Lee lecture-16 notes "工程里的关键优化点" item 3
// (K adapted to how often the draft is right).
#include "sv_rows.h"

namespace sv {

namespace {

// Softmax reference R = fp32(m*c), 1/S and kept-set threshold of one row.
struct RowStat {
  float R, invS, thr;
  int ok;
};

__device__ RowStat row_stat(const Params& P, long long unit) {
  float m, s, thr = kNegInf;
  int bad = 0;
  if (P.filt) {
    const RowRes rr = P.rowres[unit];
    m = rr.m;
    s = rr.s;
    thr = rr.theta;
    bad = rr.flags;
  } else {
    // chunk partials in chunk order (written by the previous kernel)
    m = kNegInf;
    s = 0.f;
    const unsigned long long* sl = P.slots + unit * P.chunks;
    for (int k = 0; k < P.chunks; ++k) {
      float om, os;
      unpack_ms(sl[k], om, os);
      merge_ms(m, s, om, os, P.c);
    }
  }
  RowStat r;
  r.ok = !bad && __builtin_isfinite(m) && s > 0.f && __builtin_isfinite(s);
  r.R = ref_of(m, P.c);
  r.invS = 1.0f / s;
  r.thr = thr;
  return r;
}

__device__ __forceinline__ float kept_prob(float l, const RowStat& r, float c) {
  return (l >= r.thr) ? fast_exp2(fmaf(l, c, -r.R)) * r.invS : 0.0f;
}

// Block (pair d, chunk ch): d is a draft row, its pair the target row of the
// same position.
template <int DT, bool VEC>
__global__ __launch_bounds__(kThreads) void k_beta(const Params P) {
  using Vc = Vec<DT, VEC>;
  constexpr int N = Vc::N;
  __shared__ int s_cu[kCuLds];
  __shared__ RowStat s_st[2];
  __shared__ int s_last;
  const int tid = threadIdx.x;
  const int C = P.chunks;
  const long long g = blockIdx.x;
  const int d = (int)(g / C);
  const int ch = (int)(g - (long long)d * C);
  const int b = row_seq(P, d, false, s_cu);
  const int t = d + b;  // target row of the same position
  const long long uq = unit_of(P, false, d), up = unit_of(P, true, t);
  if (tid < 2) s_st[tid] = row_stat(P, tid == 0 ? uq : up);
  __syncthreads();
  const RowStat sq = s_st[0], sp = s_st[1];
  const bool ok = sq.ok && sp.ok;
  const float c = P.c;
  float acc = 0.f;
  if (ok) {
    const size_t rq = (size_t)d * P.V, rp = (size_t)t * P.V;
    const int vb = ch * P.chunk_vecs;
    const int ve = min(P.nvec, vb + P.chunk_vecs);
    int v = vb + tid;
    for (; v + (kBatch - 1) * kThreads < ve; v += kBatch * kThreads) {
      typename Vc::Raw aq[kBatch], ap[kBatch];
#pragma unroll
      for (int u = 0; u < kBatch; ++u) {
        aq[u] = Vc::load_stream(P.draft, rq, v + u * kThreads);
        ap[u] = Vc::load_stream(P.target, rp, v + u * kThreads);
      }
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int u = 0; u < kBatch; ++u) {
        float fq[N], fp[N];
        Vc::get(aq[u], fq);
        Vc::get(ap[u], fp);
#pragma unroll
        for (int k = 0; k < N; ++k) acc += fminf(kept_prob(fp[k], sp, c), kept_prob(fq[k], sq, c));
      }
    }
    for (; v < ve; v += kThreads) {
      float fq[N], fp[N];
      Vc::get(Vc::load_stream(P.draft, rq, v), fq);
      Vc::get(Vc::load_stream(P.target, rp, v), fp);
#pragma unroll
      for (int k = 0; k < N; ++k) acc += fminf(kept_prob(fp[k], sp, c), kept_prob(fq[k], sq, c));
    }
  }
  float tot[1];
  block_sum<1>(&acc, tot);
  if (tid == 0) {
    pub_f(P.beta_part + (size_t)d * C + ch, tot[0]);
    drain_stores();
    s_last = bump(P.beta_cnt + d) == C - 1;
  }
  __syncthreads();
  if (!s_last) return;
  // Last block of the pair: the chunk sums in chunk order, then the pair's
  // partials and counter back to zero (every block of the pair has read them).
  if (tid == 0) {
    float beta = 0.f;
    for (int k = 0; k < C; ++k) beta += obs_f(P.beta_part + (size_t)d * C + k);
    P.beta[d] = ok ? beta : __builtin_nanf("");
    pub_i(P.beta_cnt + d, 0);
  }
  if (!P.filt)
    for (int k = tid; k < 2 * C; k += kThreads)
      P.slots[(k < C ? uq : up) * C + (k < C ? k : k - C)] = 0ull;
}

// Expected accepted drafts per sequence (one thread each).
__global__ __launch_bounds__(kThreads) void k_expect(const Params P) {
  const int b = blockIdx.x * kThreads + threadIdx.x;
  if (b >= P.B) return;
  int d0, kb;
  if (!seq_bounds(P, b, d0, kb)) {
    P.expected[b] = __builtin_nanf("");
    return;
  }
  float e = 0.f, run = 1.f;
  for (int i = 0; i < kb; ++i) {
    run *= P.beta[d0 + i];  // P(drafts 0..i all pass)
    e += run;
  }
  P.expected[b] = e;
}

template <int DT, bool VEC>
hipError_t launch_t(const Params& P, const Plan& L, hipStream_t s) {
  if (P.total_draft > 0) {
    hipLaunchKernelGGL((k_beta<DT, VEC>), dim3((unsigned)((long long)P.total_draft * P.chunks)),
                       dim3(kThreads), 0, s, P);
    const hipError_t err = hipGetLastError();
    if (err != hipSuccess) return err;
  }
  hipLaunchKernelGGL(k_expect, dim3((unsigned)((P.B + kThreads - 1) / kThreads)), dim3(kThreads), 0,
                     s, P);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_accept(int dtype, bool vec, const Params& P, const Plan& L, hipStream_t s) {
  switch (dtype) {
    case SV_F32:
      return vec ? launch_t<SV_F32, true>(P, L, s) : launch_t<SV_F32, false>(P, L, s);
    case SV_F16:
      return vec ? launch_t<SV_F16, true>(P, L, s) : launch_t<SV_F16, false>(P, L, s);
    default:
      return vec ? launch_t<SV_BF16, true>(P, L, s) : launch_t<SV_BF16, false>(P, L, s);
  }
}

}  // namespace sv
