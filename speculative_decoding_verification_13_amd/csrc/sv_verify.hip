// The verification step as one HIP kernel for gfx950.
//
// Grid: step s holds the stats blocks of sequence s (one per (row, V-chunk)),
// then draw chunk 0 of sequence s - lag0, then the other draw chunks of
// sequence s - lag1 (lag0 < lag1); the draws of the last sequences close the
// grid. Blocks are dispatched in index order, so when a sequence's draw chunk
// 0 starts, its stats blocks have long finished; when its other chunks start,
// chunk 0 has published the decision; and the rows being re-read were read
// recently enough to be served again from the last-level cache.
//
// Stats block (never waits): max m and sum 2^(l*c - R) of its chunk of one row
// (R = fp32(m*c)), or the chunk argmax for greedy sequences, published with one
// 64-bit agent-scope store into a slot that is zero while unpublished. It keeps
// no counter and needs no drain, so it retires as soon as its store is issued.
//
// Draw chunk 0 of sequence b decides: it reads (bounded wait) the slots of
// every row of b, merges them in chunk order, clears them, forms
// r_i = p_i(x_i)/q_i(x_i), tests u_i < r_i, finds the first rejection n, writes
// the accepted prefix and publishes the job of the final draw (residual at n,
// or the bonus row). Every draw chunk then sums the draw weights
// (max(0, p_n - q_n), or p_K) of the tiles of its part of row pair n and
// publishes them; the last one scans the sums for u*Z, re-reads that one tile,
// scans it, writes the drawn token and returns the workspace to zero.
//
// Pages (by title, section): aivaro.ru answer 289 "Как работает speculative
// decoding на уровне логитов, а не токенов?" s.5 step 3, s.6, s.9 (ratio test,
// truncation, residual max(0, p - q)/Z, multinomial draw); Hung-yi Lee
// lecture-16 notes part "4、推测解码验证流程图" items 1-4 (parallel scoring,
// position-by-position check, truncation, bonus token); aihero.vn "Speculative
// decoding" sections "Chấp nhận bằng tỉ lệ, không chỉ bằng argmax" (q draft, p
// target, ratio, residual) and "Cùng phân bố không có nghĩa cùng chuỗi mỗi lần"
// (greedy check, consistent temperature).
#include <limits.h>

#include "sv_device.h"
#include "sv_launch.h"

namespace sv {

namespace {

constexpr int kPollSlots = 2048;  // LDS staging of polled slots per group of positions

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

// ---- 64-bit slots: zero means "not published" ----
__device__ __forceinline__ void pub_u64(unsigned long long* p, unsigned long long v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ unsigned long long obs_u64(unsigned long long* p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
// (max, sum) of a sampling chunk: never all-zero bits (a +0 maximum brings a
// term 2^0 = 1 into the sum; NaN is stored canonical).
__device__ __forceinline__ unsigned long long pack_ms(float m, float s) {
  if (m != m) m = __builtin_nanf("");
  return ((unsigned long long)__float_as_uint(s) << 32) | __float_as_uint(m);
}
__device__ __forceinline__ void unpack_ms(unsigned long long v, float& m, float& s) {
  m = __uint_as_float((unsigned)v);
  s = __uint_as_float((unsigned)(v >> 32));
}
// (max value, argmax, bad flag) of a greedy chunk: the high word has bit 31 set.
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
  __device__ __forceinline__ static void get(const Raw& r, float* f) {
    if constexpr (VEC) unpack<DT>(r, f);
    else f[0] = r;
  }
};

// Weight of one id in the final draw: residual max(0, p - q) or bonus p.
__device__ __forceinline__ float draw_weight(float lp, float lq, const Job& j, float c) {
  const float ep = fast_exp2(fmaf(lp, c, -j.Rp));
  if (j.mode == kJobBonus) return ep * j.invSp;
  const float q = fast_exp2(fmaf(lq, c, -j.Rq)) * j.invSq;
  return fmaxf(fmaf(ep, j.invSp, -q), 0.0f);
}

// Block reduction of 8 values per thread; out[u] valid in every thread.
__device__ __forceinline__ void block_sum8(const float* v, float* out) {
  __shared__ float s_red[kThreads / kWave][8];
  const int lane = threadIdx.x & (kWave - 1);
  const int w = threadIdx.x / kWave;
  float t[8];
#pragma unroll
  for (int u = 0; u < 8; ++u) t[u] = wave_sum(v[u]);
  __syncthreads();
  if (lane == 0) {
#pragma unroll
    for (int u = 0; u < 8; ++u) s_red[w][u] = t[u];
  }
  __syncthreads();
#pragma unroll
  for (int u = 0; u < 8; ++u) {
    float a = 0.f;
#pragma unroll
    for (int k = 0; k < kThreads / kWave; ++k) a += s_red[k][u];
    out[u] = a;
  }
}

// First tile whose inclusive prefix exceeds u*Z (else the last tile with mass).
// Tile sums are read with agent-scope loads (published by other blocks).
__device__ __forceinline__ int find_tile(const float* ts, int ntiles, float u, float& Z,
                                         float& target, float& base) {
  __shared__ float s_base;
  const int per = (ntiles + kThreads - 1) / kThreads;
  const int t0 = threadIdx.x * per;
  const int t1 = min(ntiles, t0 + per);
  float local = 0.f;
  for (int t = t0; t < t1; ++t) local += obs_f(ts + t);
  float total;
  const float incl = block_incl_scan(local, total);
  Z = total;
  target = u * total;
  float run = incl - local;
  int cand = INT_MAX, lastpos = -1;
  for (int t = t0; t < t1; ++t) {
    const float w = obs_f(ts + t);
    const float nxt = run + w;
    if (cand == INT_MAX && nxt > target) cand = t;
    if (w > 0.f) lastpos = t;
    run = nxt;
  }
  int tile = block_min_i(cand);
  if (tile == INT_MAX) tile = block_max_i(lastpos);
  if (tile < 0) tile = 0;
  __syncthreads();
  if (tile >= t0 && tile < t1) {
    float r = incl - local;
    for (int t = t0; t < tile; ++t) r += obs_f(ts + t);
    s_base = r;
  }
  __syncthreads();
  base = s_base;
  return tile;
}

// ------------------------------------------------------------- grid mapping
// Stats blocks of sequences [0, s), s <= B: two rows (draft, target) per target
// row, `chunks` blocks per row (draft rows that do not exist stay idle).
// The grid was sized from total_draft on the host, so offsets are clamped into
// [0, total_draft] here and cu[B] is never read: the mapping always covers
// exactly the launched blocks (malformed offsets only idle some blocks).
__device__ __forceinline__ long long stats_before(const Params& P, int s) {
  long long t;
  if (P.cu == nullptr) {
    t = (long long)s * (P.K + 1);
  } else {
    const long long c = (s >= P.B) ? P.total_draft : min(max(P.cu[s], 0), P.total_draft);
    t = c + s;
  }
  return 2LL * P.chunks * t;
}
// First block of grid step s in [0, B + lag1]: stats of sequences < min(s, B),
// draw chunk 0 of sequences < s - lag0, other draw chunks of sequences < s - lag1.
__device__ __forceinline__ long long step_start(const Params& P, int s) {
  return stats_before(P, min(s, P.B)) + min(max(0, s - P.lag0), P.B) +
         (long long)(P.dchunks - 1) * min(max(0, s - P.lag1), P.B);
}

// This thread's vector of tile t (= vector t*kTileVecs + thread) of both rows.
template <int DT, bool VEC>
__device__ __forceinline__ bool tile_vector(const Params& P, const Job& j, int t, float* fp,
                                            float* fq) {
  using Vc = Vec<DT, VEC>;
  constexpr int N = Vc::N;
  const int v = t * kTileVecs + threadIdx.x;
  if (v >= P.nvec) return false;
  Vc::get(Vc::load(P.target, (size_t)j.prow * P.V, v), fp);
  if (j.mode == kJobResidual) {
    Vc::get(Vc::load(P.draft, (size_t)j.qrow * P.V, v), fq);
  } else {
#pragma unroll
    for (int k = 0; k < N; ++k) fq[k] = 0.f;
  }
  return true;
}

// Pick of the drawn token from the published tile sums (whole block).
template <int DT, bool VEC>
__device__ int pick(const Params& P, int b, Job j, float& Zout) {
  constexpr int N = Vec<DT, VEC>::N;
  float* ts = P.tiles + (size_t)b * P.ntiles;
  float Z, target, base;
  int tile = find_tile(ts, P.ntiles, j.u, Z, target, base);
  if (!(Z > 0.f) && j.mode == kJobResidual) {
    // Residual mass rounded to zero: draw from p_n instead (re-sum its tiles).
    j.mode = kJobBonus;
    __syncthreads();
    for (int t = 0; t < P.ntiles; ++t) {
      float fp[N], fq[N];
      float v[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
      if (tile_vector<DT, VEC>(P, j, t, fp, fq)) {
#pragma unroll
        for (int k = 0; k < N; ++k) v[0] += draw_weight(fp[k], fq[k], j, P.c);
      }
      float out[8];
      block_sum8(v, out);
      if (threadIdx.x == 0) pub_f(ts + t, out[0]);
    }
    drain_stores();
    __syncthreads();
    tile = find_tile(ts, P.ntiles, j.u, Z, target, base);
  }
  // Scan inside the tile: thread j owns vector tile*kTileVecs + j (ascending ids).
  float fp[N], fq[N], w[N];
  float run = 0.f;
  const int v = tile * kTileVecs + threadIdx.x;
  const bool have = tile_vector<DT, VEC>(P, j, tile, fp, fq);
#pragma unroll
  for (int k = 0; k < N; ++k) {
    if (have) run += draw_weight(fp[k], fq[k], j, P.c);
    w[k] = run;
  }
  float tot;
  const float incl = block_incl_scan(run, tot);
  const float excl = base + (incl - run);
  int cand = INT_MAX, lastpos = -1;
  float prev = 0.f;
#pragma unroll
  for (int k = 0; k < N; ++k) {
    if (cand == INT_MAX && excl + w[k] > target) cand = v * N + k;
    if (w[k] > prev) lastpos = v * N + k;
    prev = w[k];
  }
  int tok = block_min_i(cand);
  if (tok == INT_MAX) tok = block_max_i(lastpos);
  if (tok < 0) tok = tile * kTileVecs * N;
  Zout = Z;
  return tok;
}

// Per-sequence decision state, kept in LDS by the deciding block.
struct SeqState {
  float m[2][SV_MAX_K + 1];  // merged row maxima (draft, target)
  float s[2][SV_MAX_K + 1];  // merged sums 2^(l*c - R)
  int am[SV_MAX_K + 1];      // greedy argmax of target rows
  int bad[SV_MAX_K + 1];     // row not usable
  unsigned long long poll[kPollSlots];
  int flags;                 // 1 bad token, 2 bad row, 4 wait timed out
  unsigned long long rej;    // ballot of rejected draft positions
  Job job;
};

// Decision of sequence b (whole block): reads and clears the slots of its rows,
// writes the accepted prefix and the side outputs, and returns the job of the
// final draw in S.job (published for the other draw chunks when sampling).
template <int DT>
__device__ void decide(const Params& P, int b, int d0, int kb, bool greedy, SeqState& S) {
  const int tid = threadIdx.x;
  const int t0 = d0 + b;
  const bool active = tid <= kb;
  const bool is_draft = tid < kb;
  const float c = P.c;
  const int C = P.chunks;
  if (tid == 0) {
    S.flags = 0;
    S.rej = 0ull;
  }
  // inputs of the ratio test: the token and its uniform now, its logits once
  // the token is known (issued before the slot wait so the trips overlap)
  int x = -1;
  float u = 1.f;
  if (is_draft) {
    x = P.tokens[d0 + tid];
    if (!greedy) u = P.uniforms[t0 + tid];
  }
  // Read, merge (chunk order) and clear the slots, a group of positions at a time.
  const int per_pos = 2 * C;
  const int group = max(1, kPollSlots / per_pos);
  int timed_out = 0;
  for (int g0 = 0; g0 <= kb; g0 += group) {
    const int g1 = min(kb + 1, g0 + group);
    const int nslot = (g1 - g0) * per_pos;
    __syncthreads();
    for (int k = tid; k < nslot; k += kThreads) {
      const int pos = g0 + k / per_pos;
      const int which = (k % per_pos) / C;  // 0 draft row, 1 target row
      unsigned long long v = 0ull;
      if (which == 1 || (!greedy && pos < kb)) {
        unsigned long long* sl = P.slots + (size_t)(t0 + pos) * per_pos + (k % per_pos);
        int spins = 0;
        while ((v = obs_u64(sl)) == 0ull) {
          if (++spins > P.spin_limit) {
            timed_out = 1;
            break;
          }
          __builtin_amdgcn_s_sleep(2);
        }
        pub_u64(sl, 0ull);
      }
      S.poll[k] = v;
    }
    __syncthreads();
    if (tid >= g0 && tid < g1) {
      const unsigned long long* mine = S.poll + (tid - g0) * per_pos;
      if (greedy) {
        float gv = kNegInf;
        int gi = INT_MAX, gbad = 0;
        for (int k = 0; k < C; ++k) {
          float v;
          int idx, bad;
          unpack_am(mine[C + k], v, idx, bad);
          argmax_merge(gv, gi, v, idx);
          gbad |= bad;
        }
        S.m[1][tid] = gv;
        S.s[1][tid] = 0.f;
        S.am[tid] = gi;
        S.bad[tid] = gbad || gv == kNegInf;
      } else {
        float mq = kNegInf, sq = 0.f, mp = kNegInf, sp = 0.f;
        for (int k = 0; k < C; ++k) {
          float m, s;
          if (is_draft) {
            unpack_ms(mine[k], m, s);
            merge_ms(mq, sq, m, s, c);
          }
          unpack_ms(mine[C + k], m, s);
          merge_ms(mp, sp, m, s, c);
        }
        S.m[0][tid] = mq;
        S.s[0][tid] = sq;
        S.m[1][tid] = mp;
        S.s[1][tid] = sp;
        bool ok = __builtin_isfinite(mp) && sp > 0.f && __builtin_isfinite(sp);
        if (is_draft) ok = ok && __builtin_isfinite(mq) && sq > 0.f && __builtin_isfinite(sq);
        S.bad[tid] = !ok;
      }
    }
  }
  if (timed_out) atomicOr(&S.flags, 4);
  __syncthreads();
  const bool tok_ok = !is_draft || (x >= 0 && x < P.V);
  bool acc = false;
  float ratio = __builtin_nanf("");
  if (active) {
    const bool row_ok = !S.bad[tid];
    if (!row_ok) atomicOr(&S.flags, 2);
    if (!tok_ok) atomicOr(&S.flags, 1);
    if (is_draft && tok_ok && row_ok) {
      if (greedy) {
        acc = S.am[tid] == x;
      } else {
        // r = p(x)/q(x) = 2^((lp*c - Rp) - (lq*c - Rq)) * Sq / Sp
        const float lq = load_elem<DT>(P.draft, (size_t)(d0 + tid) * P.V + x);
        const float lp = load_elem<DT>(P.target, (size_t)(t0 + tid) * P.V + x);
        const float ep = fmaf(lp, c, -ref_of(S.m[1][tid], c));
        const float eq = fmaf(lq, c, -ref_of(S.m[0][tid], c));
        ratio = fast_exp2(ep - eq) * (S.s[0][tid] / S.s[1][tid]);
        acc = u < ratio;  // strict: u == r rejects
      }
    }
  }
  if (tid < kWave) {
    const unsigned long long rej = __ballot(is_draft && !acc);
    if (tid == 0) S.rej = rej;
  }
  __syncthreads();
  const int sf = S.flags;
  const int code = (sf & 1) ? SV_SEQ_BAD_TOKEN
                            : ((sf & 2) ? SV_SEQ_BAD_ROW : ((sf & 4) ? SV_SEQ_SYNC_TIMEOUT : 0));
  const int n = S.rej ? (__ffsll(S.rej) - 1) : kb;
  const bool draws = code == 0 && !greedy;

  // outputs: slot n of a drawing sequence belongs to the draw chunks
  if (active && !(draws && tid == n)) {
    int tok = -1;
    if (code == 0) {
      if (tid < n) tok = x;
      else if (tid == n) tok = S.am[n];
    }
    P.out_tokens[t0 + tid] = tok;
  }
  const float kLn2 = 0.69314718055994531f;
  const float nan = __builtin_nanf("");
  if (active) {
    const float mp = S.m[1][tid], sp = S.s[1][tid];
    if (P.diag.row_max_target) P.diag.row_max_target[t0 + tid] = mp;
    if (P.diag.row_logsum_target)
      P.diag.row_logsum_target[t0 + tid] =
          greedy ? nan : (__log2f(sp) + fmaf(-mp, c, ref_of(mp, c))) * kLn2;
    if (is_draft) {
      const float mq = S.m[0][tid], sq = S.s[0][tid];
      if (P.diag.row_max_draft) P.diag.row_max_draft[d0 + tid] = greedy ? nan : mq;
      if (P.diag.row_logsum_draft)
        P.diag.row_logsum_draft[d0 + tid] =
            greedy ? nan : (__log2f(sq) + fmaf(-mq, c, ref_of(mq, c))) * kLn2;
      if (P.diag.ratio) P.diag.ratio[d0 + tid] = ratio;
    }
  }
  if (tid == 0) {
    if (!draws) {
      P.num_accepted[b] = code ? code : n;
      if (P.diag.resid_Z) P.diag.resid_Z[b] = nan;
    }
    Job j;
    j.mode = draws ? (n < kb ? kJobResidual : kJobBonus) : kJobNone;
    j.n = n;
    j.prow = t0 + n;
    j.qrow = d0 + n;
    j.Rq = ref_of(S.m[0][n], c);
    j.invSq = 1.0f / S.s[0][n];
    j.Rp = ref_of(S.m[1][n], c);
    j.invSp = 1.0f / S.s[1][n];
    j.u = draws ? P.uniforms[t0 + kb] : 0.f;
    j.out_idx = t0 + n;
    S.job = j;
    if (!greedy) {
      int* q = reinterpret_cast<int*>(P.jobs + b);
      pub_i(q, j.mode);
      pub_i(q + 1, j.n);
      pub_i(q + 2, j.prow);
      pub_i(q + 3, j.qrow);
      pub_f(reinterpret_cast<float*>(q + 4), j.Rq);
      pub_f(reinterpret_cast<float*>(q + 5), j.invSq);
      pub_f(reinterpret_cast<float*>(q + 6), j.Rp);
      pub_f(reinterpret_cast<float*>(q + 7), j.invSp);
      pub_f(reinterpret_cast<float*>(q + 8), j.u);
      pub_i(q + 9, j.out_idx);
      drain_stores();
      pub_i(P.job_ready + b, 1);
    }
  }
  __syncthreads();
}

// Bounded wait (one thread) until *flag != 0. Returns false on timeout.
__device__ __forceinline__ bool wait_flag(const Params& P, const int* flag) {
  int spins = 0;
  while (obs_i(flag) == 0) {
    if (++spins > P.spin_limit) return false;
    __builtin_amdgcn_s_sleep(8);
  }
  compiler_fence();
  return true;
}

// ----------------------------------------------------------------- stats block
template <int DT, bool VEC>
__device__ void stats_block(const Params& P, int b, int d0, int kb, int local, int ch) {
  using Vc = Vec<DT, VEC>;
  constexpr int N = Vc::N;
  __shared__ float4 s_part[kThreads / kWave];
  const int tid = threadIdx.x;
  const int lane = tid & (kWave - 1);
  const int wave = tid / kWave;
  const int i = local >> 1;
  const int which = local & 1;  // 0: draft row of position i, 1: target row
  const int rp = d0 + b + i;
  const bool greedy = seq_greedy(P, b);
  if (which == 0 && (greedy || i == kb)) return;  // no draft row to read
  const void* base = which ? P.target : P.draft;
  const size_t row = (size_t)(which ? rp : d0 + i) * (size_t)P.V;
  const int vb = ch * kChunkVecs;
  const int ve = min(P.nvec, vb + kChunkVecs);
  int v = vb + tid;
  unsigned long long packed;
  if (greedy) {
    float bv = kNegInf;
    int bi = INT_MAX, bad = 0;
    for (; v + (kBatch - 1) * kThreads < ve; v += kBatch * kThreads) {
      typename Vc::Raw r[kBatch];
#pragma unroll
      for (int u = 0; u < kBatch; ++u) r[u] = Vc::load(base, row, v + u * kThreads);
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
      Vc::get(Vc::load(base, row, v), f);
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
    if (tid != 0) return;
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
#pragma unroll
      for (int u = 0; u < kBatch; ++u) r[u] = Vc::load(base, row, v + u * kThreads);
      __builtin_amdgcn_sched_barrier(0);
      float f[kBatch * N];
#pragma unroll
      for (int u = 0; u < kBatch; ++u) Vc::get(r[u], f + u * N);
      online_update<kBatch * N>(m, s, f, c);
    }
    for (; v < ve; v += kThreads) {
      float f[N];
      Vc::get(Vc::load(base, row, v), f);
      online_update<N>(m, s, f, c);
    }
    wave_merge_ms(m, s, c);
    if (lane == 0) s_part[wave] = make_float4(m, s, 0.f, 0.f);
    __syncthreads();
    if (tid != 0) return;
#pragma unroll
    for (int w = 1; w < kThreads / kWave; ++w) merge_ms(m, s, s_part[w].x, s_part[w].y, c);
    packed = pack_ms(m, s);
  }
  pub_u64(P.slots + ((size_t)rp * 2 + which) * P.chunks + ch, packed);
}

// ------------------------------------------------------------------ draw block
template <int DT, bool VEC>
__device__ void draw_block(const Params& P, int b, int ch) {
  using Vc = Vec<DT, VEC>;
  constexpr int N = Vc::N;
  __shared__ SeqState S;
  __shared__ int s_last, s_to;
  const int tid = threadIdx.x;
  int d0, kb;
  if (!seq_bounds(P, b, d0, kb)) return;  // reported by the offsets check
  const bool greedy = seq_greedy(P, b);
  if (greedy) {
    // chunk 0 decides a greedy sequence; there is nothing to draw
    if (ch == 0) decide<DT>(P, b, d0, kb, true, S);
    return;
  }
  if (ch == 0) {
    decide<DT>(P, b, d0, kb, false, S);
  } else {
    if (tid == 0) {
      const bool ok = wait_flag(P, P.job_ready + b);
      Job j;
      const int* q = reinterpret_cast<const int*>(P.jobs + b);
      j.mode = ok ? obs_i(q) : kJobNone;
      j.n = obs_i(q + 1);
      j.prow = obs_i(q + 2);
      j.qrow = obs_i(q + 3);
      j.Rq = obs_f(reinterpret_cast<const float*>(q + 4));
      j.invSq = obs_f(reinterpret_cast<const float*>(q + 5));
      j.Rp = obs_f(reinterpret_cast<const float*>(q + 6));
      j.invSp = obs_f(reinterpret_cast<const float*>(q + 7));
      j.u = obs_f(reinterpret_cast<const float*>(q + 8));
      j.out_idx = obs_i(q + 9);
      if (!ok) {
        raise_flag(P.seq_flags + b, kSeqFlagTimeout);
        drain_stores();
      }
      S.job = j;
    }
    __syncthreads();
  }
  const Job j = S.job;
  if (j.mode != kJobNone) {
    // tile sums of this draw chunk of row pair n: the thread's vector
    // k*kThreads + tid of the chunk belongs to tile ch*kTilesPerDraw + k
    const size_t prow = (size_t)j.prow * P.V;
    const size_t qrow = (size_t)j.qrow * P.V;
    const int vb = ch * kDrawVecs + tid;
    typename Vc::Raw rp[kBatch], rq[kBatch];
#pragma unroll
    for (int u = 0; u < kBatch; ++u) {
      const int v = vb + u * kThreads;
      if (v < P.nvec) {
        rp[u] = Vc::load(P.target, prow, v);
        if (j.mode == kJobResidual) rq[u] = Vc::load(P.draft, qrow, v);
      }
    }
    __builtin_amdgcn_sched_barrier(0);
    float ts[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int u = 0; u < kBatch; ++u) {
      const int v = vb + u * kThreads;
      if (v < P.nvec) {
        float fp[N], fq[N];
        Vc::get(rp[u], fp);
        if (j.mode == kJobResidual) Vc::get(rq[u], fq);
        float s = 0.f;
#pragma unroll
        for (int k = 0; k < N; ++k) s += draw_weight(fp[k], fq[k], j, P.c);
        ts[u] = s;
      }
    }
    float tot[8];
    block_sum8(ts, tot);
    if (tid < kTilesPerDraw) {
      float val = tot[0];
#pragma unroll
      for (int k = 1; k < kTilesPerDraw; ++k) val = (tid == k) ? tot[k] : val;
      pub_f(P.tiles + (size_t)b * P.ntiles + ch * kTilesPerDraw + tid, val);
      drain_stores();
    }
  }
  // every draw chunk of the sequence counts itself, timed out or not
  __syncthreads();
  if (tid == 0) {
    s_last = (bump(P.draw_done + b) == P.dchunks - 1) ? 1 : 0;
    compiler_fence();
  }
  __syncthreads();
  if (!s_last) return;
  // Last draw chunk: draw, write the token, return the workspace to zero.
  if (tid == 0) s_to = obs_i(P.seq_flags + b) & kSeqFlagTimeout;
  __syncthreads();
  if (s_to) {
    for (int k = tid; k <= kb; k += kThreads) P.out_tokens[d0 + b + k] = -1;
    if (tid == 0) P.num_accepted[b] = SV_SEQ_SYNC_TIMEOUT;
  } else if (j.mode != kJobNone) {
    float Z;
    const int tok = pick<DT, VEC>(P, b, j, Z);
    if (tid == 0) {
      P.out_tokens[j.out_idx] = tok;
      P.num_accepted[b] = j.n;
      if (P.diag.resid_Z) P.diag.resid_Z[b] = Z;
    }
  }
  __syncthreads();
  if (j.mode != kJobNone)
    for (int t = tid; t < P.ntiles; t += kThreads) pub_f(P.tiles + (size_t)b * P.ntiles + t, 0.f);
  if (tid < (int)(sizeof(Job) / sizeof(int))) pub_i(reinterpret_cast<int*>(P.jobs + b) + tid, 0);
  if (tid == 0) {
    pub_i(P.job_ready + b, 0);
    pub_i(P.draw_done + b, 0);
    pub_i(P.seq_flags + b, 0);
  }
}

}  // namespace

template <int DT, bool VEC>
__global__ __launch_bounds__(kThreads) void k_verify(const Params P) {
  // Sequences whose own offsets are invalid are reported by block b.
  if (P.cu != nullptr && blockIdx.x < (unsigned)P.B && threadIdx.x == 0) {
    int d0_, kb_;
    if (!seq_bounds(P, blockIdx.x, d0_, kb_)) P.num_accepted[blockIdx.x] = SV_SEQ_BAD_OFFSETS;
  }
  // step s of the grid: stats blocks of sequence s, draw chunk 0 of s - lag0,
  // the other draw chunks of s - lag1
  const long long idx = blockIdx.x;
  int lo = 0, hi = P.B + P.lag1 - 1;
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (step_start(P, mid) <= idx) lo = mid;
    else hi = mid - 1;
  }
  const int step = lo;
  long long off = idx - step_start(P, step);
  int d0, kb;
  long long nstats = 0;
  if (step < P.B && seq_bounds(P, step, d0, kb)) nstats = 2LL * P.chunks * (kb + 1);
  const long long nstats_slots =
      (step < P.B) ? stats_before(P, step + 1) - stats_before(P, step) : 0;
  if (off < nstats) {
    stats_block<DT, VEC>(P, step, d0, kb, (int)(off / P.chunks), (int)(off % P.chunks));
    return;
  }
  off -= nstats_slots;
  if (off < 0) return;  // idle block of a sequence with invalid offsets
  const int b0 = step - P.lag0;
  if (b0 >= 0 && b0 < P.B) {
    if (off == 0) {
      draw_block<DT, VEC>(P, b0, 0);
      return;
    }
    off -= 1;
  }
  const int b1 = step - P.lag1;
  if (b1 >= 0 && b1 < P.B && off < P.dchunks - 1) draw_block<DT, VEC>(P, b1, (int)off + 1);
}

__global__ void k_fill_zero(uint4* p, size_t n16) {
  for (size_t k = (size_t)blockIdx.x * blockDim.x + threadIdx.x; k < n16;
       k += (size_t)gridDim.x * blockDim.x)
    p[k] = make_uint4(0, 0, 0, 0);
}

template <int DT, bool VEC>
static hipError_t launch_t(const Params& P, const Plan& L, hipStream_t s, hipEvent_t* ev, int nev) {
  hipError_t err;
  if (ev != nullptr && nev > 0 && (err = hipEventRecord(ev[0], s)) != hipSuccess) return err;
  hipLaunchKernelGGL((k_verify<DT, VEC>), dim3((unsigned)L.blocks), dim3(kThreads), 0, s, P);
  if ((err = hipGetLastError()) != hipSuccess) return err;
  if (ev != nullptr && nev > 1 && (err = hipEventRecord(ev[1], s)) != hipSuccess) return err;
  return hipSuccess;
}

hipError_t launch(int dtype, bool vec, const Params& P, const Plan& L, hipStream_t s,
                  hipEvent_t* ev, int nev) {
  switch (dtype) {
    case SV_F32:
      return vec ? launch_t<SV_F32, true>(P, L, s, ev, nev) : launch_t<SV_F32, false>(P, L, s, ev, nev);
    case SV_F16:
      return vec ? launch_t<SV_F16, true>(P, L, s, ev, nev) : launch_t<SV_F16, false>(P, L, s, ev, nev);
    default:
      return vec ? launch_t<SV_BF16, true>(P, L, s, ev, nev) : launch_t<SV_BF16, false>(P, L, s, ev, nev);
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
