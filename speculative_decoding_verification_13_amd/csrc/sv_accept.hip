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
// zero, and the last pair of a sequence to finish forms its E[n].
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

// Softmax reference R = fp32(m*c), sum S of 2^(l*c - R) over the kept set and
// kept-set threshold of one row: p(x) = 2^(l*c - R) / S for kept ids.
struct RowStat {
  float R, S, thr;
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
  r.S = s;
  r.thr = thr;
  return r;
}

constexpr int kBetaBatch = 4;  // vectors per row per thread in flight (2 to 8 measured alike)
constexpr int kBetaWaves = 7;  // waves per SIMD asked of the compiler

// l*c - R of a logit, -inf outside the kept set.
template <bool FILT>
__device__ __forceinline__ float rel_exp(float l, float c, float R, float thr) {
  const float x = fmaf(l, c, -R);
  if constexpr (FILT) return (l >= thr) ? x : kNegInf;
  return x;
}

// Expected accepted drafts of sequence b from its published pass
// probabilities: sum_{j<K_b} prod_{i<=j} beta_i (NaN for invalid offsets).
__device__ void write_expected(const Params& P, int b) {
  int d0, kb;
  if (!seq_bounds(P, b, d0, kb)) {
    P.expected[b] = __builtin_nanf("");
    return;
  }
  float e = 0.f, run = 1.f;
  for (int i = 0; i < kb; ++i) {
    run *= obs_f(P.beta + d0 + i);  // P(drafts 0..i all pass)
    e += run;
  }
  P.expected[b] = e;
}

// Block (pair d, chunk ch): d is a draft row, its pair the target row of the
// same position. With a = l_p*c - R_p, b = l_q*c - R_q and
// delta = log2(S_q / S_p): min(p, q) = 2^min(a, b - delta) / S_p, one
// exponential per pair of logits (the offsets stay small, so each term keeps
// the precision of its own row's exponent).
template <int DT, bool VEC, bool FILT>
__global__ __launch_bounds__(kThreads, kBetaWaves) void k_beta(const Params P) {
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
  if (g == 0 && P.cu != nullptr) {
    // sequences without pairs: no draft (expected 0) or invalid offsets (NaN)
    for (int k = tid; k < P.B; k += kThreads) {
      int d0, kb;
      if (!seq_bounds(P, k, d0, kb)) P.expected[k] = __builtin_nanf("");
      else if (kb == 0) P.expected[k] = 0.f;
    }
  }
  if (tid < 2) s_st[tid] = row_stat(P, tid == 0 ? uq : up);
  __syncthreads();
  const RowStat sq = s_st[0], sp = s_st[1];
  const bool ok = sq.ok && sp.ok;
  const float c = P.c;
  const float delta = __log2f(sq.S / sp.S);
  float acc = 0.f;
  if (ok) {
    const size_t rq = (size_t)d * P.V, rp = (size_t)t * P.V;
    const int vb = ch * P.chunk_vecs;
    const int ve = min(P.nvec, vb + P.chunk_vecs);
    int v = vb + tid;
    for (; v + (kBetaBatch - 1) * kThreads < ve; v += kBetaBatch * kThreads) {
      typename Vc::Raw aq[kBetaBatch], ap[kBetaBatch];
#pragma unroll
      for (int u = 0; u < kBetaBatch; ++u) {
        aq[u] = Vc::load_stream(P.draft, rq, v + u * kThreads);
        ap[u] = Vc::load_stream(P.target, rp, v + u * kThreads);
      }
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int u = 0; u < kBetaBatch; ++u) {
        float fq[N], fp[N];
        Vc::get(aq[u], fq);
        Vc::get(ap[u], fp);
#pragma unroll
        for (int k = 0; k < N; ++k)
          acc += fast_exp2(fminf(rel_exp<FILT>(fp[k], c, sp.R, sp.thr),
                                 rel_exp<FILT>(fq[k], c, sq.R, sq.thr) - delta));
      }
    }
    for (; v < ve; v += kThreads) {
      float fq[N], fp[N];
      Vc::get(Vc::load_stream(P.draft, rq, v), fq);
      Vc::get(Vc::load_stream(P.target, rp, v), fp);
#pragma unroll
      for (int k = 0; k < N; ++k)
        acc += fast_exp2(fminf(rel_exp<FILT>(fp[k], c, sp.R, sp.thr),
                               rel_exp<FILT>(fq[k], c, sq.R, sq.thr) - delta));
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
  // chunk sums, partials and counter back to zero (every block of the pair
  // has read the partials);
  // the last pair of the sequence forms the expected count.
  if (tid == 0) {
    float beta = 0.f;
    for (int k = 0; k < C; ++k) {
      beta += obs_f(P.beta_part + (size_t)d * C + k);
      P.beta_part[(size_t)d * C + k] = 0.f;
    }
    pub_f(P.beta + d, ok ? beta / sp.S : __builtin_nanf(""));
    pub_i(P.beta_cnt + d, 0);
    drain_stores();
    int d0, kb;
    const int need = seq_bounds(P, b, d0, kb) ? kb : 1;
    if (bump(P.draw_done + b) == need - 1) {
      pub_i(P.draw_done + b, 0);
      write_expected(P, b);
    }
  }
  if (!P.filt) {
    for (int k = tid; k < 2 * C; k += kThreads)
      P.slots[(k < C ? uq : up) * C + (k < C ? k : k - C)] = 0ull;
  } else if (tid < 2) {
    P.rowres[tid == 0 ? uq : up] = RowRes{0.f, 0.f, 0.f, 0};  // every block has read it
  }
}

// Expected accepted drafts when the batch has no draft rows (every sequence 0,
// or NaN for invalid offsets).
__global__ __launch_bounds__(kThreads) void k_expect(const Params P) {
  const int b = blockIdx.x * kThreads + threadIdx.x;
  if (b < P.B) write_expected(P, b);
}

template <int DT, bool VEC>
hipError_t launch_t(const Params& P, const Plan& L, hipStream_t s) {
  const dim3 grid((unsigned)((long long)P.total_draft * P.chunks));
  if (P.total_draft == 0)
    hipLaunchKernelGGL(k_expect, dim3((unsigned)((P.B + kThreads - 1) / kThreads)), dim3(kThreads),
                       0, s, P);
  else if (P.filt)
    hipLaunchKernelGGL((k_beta<DT, VEC, true>), grid, dim3(kThreads), 0, s, P);
  else
    hipLaunchKernelGGL((k_beta<DT, VEC, false>), grid, dim3(kThreads), 0, s, P);
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
