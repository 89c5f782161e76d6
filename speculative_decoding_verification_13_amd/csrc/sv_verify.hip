// The verification step as separate statistics, filter and draw kernels for
// gfx950: the path of calls with top-k / top-p filters, and of unfiltered calls
// whose rows are too long for the one-kernel step (sv_fused.hip).
//
// k_stats streams every logit row once. Each block takes one chunk of one row
// and writes one 64-bit partial: for a sampling row the chunk maximum m and the
// sum of 2^(l*c - R) with R = fp32(m*c); for a greedy row the chunk argmax
// (lowest id on ties) and whether the chunk holds NaN or +inf. Blocks never
// wait on each other; the kernel boundary publishes the partials.
//
// With filters a per-row pass sits between them: k_filter (top-k, then top-p)
// selects the row's k-th largest logit from the chunks' candidate records and
// applies the top-p cut to the levels above it; k_nucleus (top-p alone) finds
// the cut by a radix descent over the whole row. Both leave the row's kept-set
// threshold and normaliser.
//
// k_draw runs one group of blocks per sequence, each group covering the vocabulary
// of one row pair in slices. Every block of the group merges the row partials
// of its sequence in chunk order, forms r_i = p_i(x_i)/q_i(x_i), tests
// u_i < r_i and finds the first rejection n itself (the same arithmetic in
// every block gives the same decision, so no block waits for another). Each
// block then sums the draw weights (max(0, p_n - q_n), or p_K for the bonus)
// over the tiles of its slice and publishes the sums; the last block of the
// group to finish scans the tile sums for u*Z, re-reads the one tile that
// holds the crossing, scans it and writes the drawn token.
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

#include "sv_rows.h"

namespace sv {

namespace {

// NaN-propagating maximum of one register-held vector: packed over fp16
// pairs, over widened values otherwise.
template <int DT, bool VEC, class Raw>
__device__ __forceinline__ float vec_max_prop(const Raw& w) {
  if constexpr (VEC && DT == SV_F16) {
    const half2_t a = __builtin_bit_cast(half2_t, w.x), b = __builtin_bit_cast(half2_t, w.y);
    const half2_t cc = __builtin_bit_cast(half2_t, w.z), d = __builtin_bit_cast(half2_t, w.w);
    const half2_t m2 = __builtin_elementwise_maximum(__builtin_elementwise_maximum(a, b),
                                                     __builtin_elementwise_maximum(cc, d));
    return __builtin_elementwise_maximum((float)m2.x, (float)m2.y);
  } else {
    constexpr int N = VEC ? Dt<DT>::N : 1;
    float f[N];
    Vec<DT, VEC>::get(w, f);
    float m = f[0];
#pragma unroll
    for (int k = 1; k < N; ++k) m = __builtin_elementwise_maximum(m, f[k]);
    return m;
  }
}

// First tile whose inclusive prefix exceeds u*Z (else the last tile with mass).
// Tile sums are read once with agent-scope loads (published by other blocks);
// a thread's first kTileKeep sums stay in registers for the second walk.
__device__ __forceinline__ int find_tile(const float* ts, int ntiles, float u, float& Z,
                                         float& target, float& base) {
  constexpr int kTileKeep = 4;
  __shared__ float s_base;
  const int per = (ntiles + kThreads - 1) / kThreads;
  const int t0 = threadIdx.x * per;
  const int t1 = min(ntiles, t0 + per);
  float keep[kTileKeep];
  float local = 0.f;
#pragma unroll
  for (int q = 0; q < kTileKeep; ++q) {
    keep[q] = (t0 + q < t1) ? obs_f(ts + t0 + q) : 0.f;
    local += keep[q];
  }
  for (int t = t0 + kTileKeep; t < t1; ++t) local += obs_f(ts + t);
  float total;
  const float incl = block_incl_scan(local, total);
  Z = total;
  target = u * total;
  float run = incl - local;
  int cand = INT_MAX, lastpos = -1;
  for (int t = t0; t < t1; ++t) {
    float w = 0.f;
#pragma unroll
    for (int q = 0; q < kTileKeep; ++q) w = (t == t0 + q) ? keep[q] : w;
    if (t >= t0 + kTileKeep) w = obs_f(ts + t);
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
    for (int t = t0; t < tile; ++t) {
      float w = 0.f;
#pragma unroll
      for (int q = 0; q < kTileKeep; ++q) w = (t == t0 + q) ? keep[q] : w;
      if (t >= t0 + kTileKeep) w = obs_f(ts + t);
      r += w;
    }
    s_base = r;
  }
  __syncthreads();
  base = s_base;
  return tile;
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

// Decision state of one sequence, in LDS.
struct Dec {
  float m[2][SV_MAX_K + 1];  // merged row maxima (draft, target) per position
  float s[2][SV_MAX_K + 1];  // merged sums 2^(l*c - R) (over the kept set)
  float th[2][SV_MAX_K + 1]; // kept-set thresholds (-inf: no filter)
  int flags;                 // 1 a draft id outside [0, V)
  int first;                 // first position that stops the walk (rejection,
                             // invalid row or id, or the bonus position)
  int invalid;               // first position with an invalid row
};

// Merge the chunk partials of one position's rows in chunk order (loads issued
// four chunks at a time so their round trips overlap). The partials were
// written by an earlier kernel.
__device__ __forceinline__ void merge_sampling(const unsigned long long* dsl,
                                               const unsigned long long* tsl, bool with_draft,
                                               int C, float c, float& mq, float& sq, float& mp,
                                               float& sp) {
  constexpr int G = 4;
  for (int k0 = 0; k0 < C; k0 += G) {
    unsigned long long dv[G], tv[G];
#pragma unroll
    for (int g = 0; g < G; ++g) {
      const bool in = k0 + g < C;
      tv[g] = in ? tsl[k0 + g] : 1ull;
      dv[g] = (in && with_draft) ? dsl[k0 + g] : 1ull;
    }
#pragma unroll
    for (int g = 0; g < G; ++g) {
      if (k0 + g < C) {
        float m, s;
        if (with_draft) {
          unpack_ms(dv[g], m, s);
          merge_ms(mq, sq, m, s, c);
        }
        unpack_ms(tv[g], m, s);
        merge_ms(mp, sp, m, s, c);
      }
    }
  }
}


// Decision of sequence b (whole block; thread i owns position i). Position i
// stops the walk if a row it reads is invalid, its draft id is out of range or
// its ratio test rejects; the bonus position always stops. n is the first
// stopping position. The row statistics come from an earlier kernel. Every
// block of the sequence computes the same result; only the writer block stores
// the outputs it fixes: the accepted prefix and -1 after it, the side outputs,
// and num_accepted when nothing is drawn. Returns the job of the final draw
// (kJobNone when there is none).
template <int DT>
__device__ Job decide(const Params& P, int b, int d0, int kb, bool greedy, bool writer, Dec& S) {
  const int tid = threadIdx.x;
  const int t0 = d0 + b;
  const bool active = tid <= kb;
  const bool is_draft = tid < kb;
  const float c = P.c;
  const int C = P.chunks;
  if (tid == 0) {
    S.flags = 0;
    S.first = kb + 1;
    S.invalid = INT_MAX;
  }
  __syncthreads();
  const unsigned long long* tsl = P.slots + unit_of(P, true, t0 + min(tid, kb)) * C;
  const unsigned long long* dsl = is_draft ? P.slots + unit_of(P, false, d0 + tid) * C : tsl;
  int x = -1;
  float u = 1.f;
  if (is_draft) {
    x = P.tokens[d0 + tid];
    if (!greedy) u = P.uniforms[t0 + tid];
  }
  const float u_draw = greedy ? 0.f : P.uniforms[t0 + kb];
  const bool tok_ok = !is_draft || (x >= 0 && x < P.V);
  // logits at the draft token (issued before the partials are merged)
  float lq = 0.f, lp = 0.f;
  if (is_draft && !greedy) {
    const int xs = tok_ok ? x : 0;
    if (P.tok_logits != nullptr) {
      lq = P.tok_logits[unit_of(P, false, d0 + tid)];
      lp = P.tok_logits[unit_of(P, true, t0 + tid)];
    } else {
      lq = load_elem<DT>(P.draft, (size_t)(d0 + tid) * P.V + xs);
      lp = load_elem<DT>(P.target, (size_t)(t0 + tid) * P.V + xs);
    }
  }
  if (!tok_ok) atomicOr(&S.flags, 1);  // every draft id is checked
  float mq = kNegInf, sq = 0.f, mp = kNegInf, sp = 0.f;
  float thq = kNegInf, thp = kNegInf;
  int am = INT_MAX;
  bool valid = false, acc = false;
  float ratio = __builtin_nanf("");
  if (active) {
    if (greedy) {
      int gbad = 0;
      merge_greedy(tsl, C, mp, am, gbad);
      valid = !gbad && mp != kNegInf;
    } else {
      int rbad = 0;
      if (P.filt) {
        // kept-set statistics of the filter pass
        const RowRes rt = P.rowres[P.total_draft + t0 + tid];
        mp = rt.m;
        sp = rt.s;
        thp = rt.theta;
        rbad = rt.flags;
        if (is_draft) {
          const RowRes rd = P.rowres[d0 + tid];
          mq = rd.m;
          sq = rd.s;
          thq = rd.theta;
          rbad |= rd.flags;
        }
      } else {
        merge_sampling(dsl, tsl, is_draft, C, c, mq, sq, mp, sp);
      }
      valid = !rbad && __builtin_isfinite(mp) && sp > 0.f && __builtin_isfinite(sp);
      if (is_draft) valid = valid && __builtin_isfinite(mq) && sq > 0.f && __builtin_isfinite(sq);
    }
    if (is_draft && tok_ok && valid) {
      if (greedy) {
        acc = am == x;
      } else {
        // r = p(x)/q(x) = 2^((lp*c - Rp) - (lq*c - Rq)) * Sq / Sp; an id
        // outside a row's kept set has probability 0 there: q(x) = 0 < p(x)
        // accepts, p(x) = 0 rejects
        const bool pk = lp >= thp, qk = lq >= thq;
        if (pk && qk) {
          const float ep = fmaf(lp, c, -ref_of(mp, c));
          const float eq = fmaf(lq, c, -ref_of(mq, c));
          ratio = fast_exp2(ep - eq) * (sq / sp);
        } else {
          ratio = pk ? kPosInf : 0.f;
        }
        acc = u < ratio;  // strict: u == r rejects
      }
    }
    if (!valid) atomicMin(&S.invalid, tid);
    if (!acc) atomicMin(&S.first, tid);  // also the bonus position and bad ids
    S.m[0][tid] = mq;
    S.s[0][tid] = sq;
    S.m[1][tid] = mp;
    S.s[1][tid] = sp;
    S.th[0][tid] = thq;
    S.th[1][tid] = thp;
  }
  __syncthreads();
  const int first = S.first;
  const int n = min(first, kb);
  const int code = (S.flags & 1) ? SV_SEQ_BAD_TOKEN : (S.invalid == n) ? SV_SEQ_BAD_ROW : 0;
  const bool draws = code == 0 && !greedy;

  if (writer) {
    // slot n of a drawing sequence is written by the block that draws. Outputs
    // another block may overwrite later (a timed-out wait) are written with
    // agent-scope stores, so they reach the coherence point before this block
    // counts itself and the later overwrite lands after them.
    if (active && !(draws && tid == n)) {
      int tok = -1;
      if (code == 0) {
        if (tid < n) tok = x;
        else if (tid == n) tok = am;
      }
      pub_i(P.out_tokens + t0 + tid, tok);
    }
    const float kLn2 = 0.69314718055994531f;
    const float nan = __builtin_nanf("");
    if (active) {
      if (P.diag.row_max_target) P.diag.row_max_target[t0 + tid] = mp;
      if (P.diag.row_logsum_target)
        P.diag.row_logsum_target[t0 + tid] =
            greedy ? nan : (__log2f(sp) + fmaf(-mp, c, ref_of(mp, c))) * kLn2;
      if (is_draft) {
        if (P.diag.row_max_draft) P.diag.row_max_draft[d0 + tid] = greedy ? nan : mq;
        if (P.diag.row_logsum_draft)
          P.diag.row_logsum_draft[d0 + tid] =
              greedy ? nan : (__log2f(sq) + fmaf(-mq, c, ref_of(mq, c))) * kLn2;
        if (P.diag.ratio) P.diag.ratio[d0 + tid] = ratio;
      }
    }
    if (tid == 0 && !draws) {
      pub_i(P.num_accepted + b, code ? code : n);
      if (P.diag.resid_Z) pub_f(P.diag.resid_Z + b, nan);
    }
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
  j.thr_q = S.th[0][n];
  j.thr_p = S.th[1][n];
  j.u = u_draw;
  j.out_idx = t0 + n;
  return j;
}


// Candidates of one chunk of a filtered sampling row (whole block; the chunk
// stays in registers). The candidates are the finite logits at or above a
// lower bound of the chunk's k-th largest finite logit, so they include every
// logit the row's top-k set can take from this chunk. They are written to the
// chunk record as (value bits, id) pairs. Only vectors whose maximum reaches
// the bound hold candidates: those few are staged in LDS and examined there,
// so the per-logit work is one maximum. A chunk with more candidates than the
// record holds (heavy ties, or k beyond what the bound covers) is cut to its
// exact top k by a radix select on order-preserving keys; a tie class at the
// cut that still does not fit is recorded as (value, count). Header word 4
// holds a lower bound of the chunk's k-th largest finite logit (-FLT_MAX when
// the chunk gives none): every logit at or above it is in the record.
template <int DT, bool VEC>
__device__ void topk_block(const Params& P, long long g, const void* base, size_t roff, int ch) {
  using Vc = Vec<DT, VEC>;
  constexpr int N = Vc::N;
  __shared__ __align__(16) float s_max[kThreads];
  __shared__ int s_hist[256];
  __shared__ int s_sel[2];
  const int tid = threadIdx.x;
  const int vb = ch * P.chunk_vecs;
  typename Vc::Raw r[kFiltVpt]{};
#pragma unroll
  for (int u = 0; u < kFiltVpt; ++u) {
    const int v = vb + u * kThreads + tid;
    if (v < P.nvec) r[u] = Vc::load_stream(base, roff, v);
  }
  // The rare paths below (invalid chunks, k beyond the bound, more
  // candidates than the record holds) visit this thread's logits again in
  // ascending id order, re-reading them one vector at a time so that the
  // registers above are free by then: fn(value, id).
  auto each = [&](auto&& fn) {
#pragma unroll 1
    for (int u = 0; u < kFiltVpt; ++u) {
      const int v = vb + u * kThreads + tid;
      if (v < P.nvec) {
        float f[N];
        Vc::get(Vc::load(base, roff, v), f);
#pragma unroll
        for (int k = 0; k < N; ++k) fn(f[k], v * N + k);
      }
    }
  };
  // Vector and thread maxima with a NaN-propagating max: a NaN or +inf
  // anywhere in the thread's logits shows up as the maximum (-inf does not).
  float vm[kFiltVpt];
#pragma unroll
  for (int u = 0; u < kFiltVpt; ++u)
    vm[u] = (vb + u * kThreads + tid < P.nvec) ? vec_max_prop<DT, VEC>(r[u]) : kNegInf;
  float tmax = vm[0];
#pragma unroll
  for (int u = 1; u < kFiltVpt; ++u) tmax = __builtin_elementwise_maximum(tmax, vm[u]);
  const int bad = (tmax != tmax || tmax == kPosInf) ? 1 : 0;
  // Bound: with the threads in groups of g (g = 4, 2 or 1, the largest with
  // at least k groups), the largest group maximum that at least k group maxima
  // reach; k groups then hold a finite logit >= it, so it is <= the chunk's
  // k-th largest. Only the threads that own a group count.
  const int k = P.top_k;
  __shared__ unsigned s_lbk;  // the bound as an order-preserving key
  float lb = kNegInf;
  if (k <= kBoundMaxK) {
    const int g = (k <= kThreads / 4) ? 4 : ((k <= kThreads / 2) ? 2 : 1);
    float gm = tmax;
    if (g >= 2) gm = fmaxf(gm, dpp_f<0xB1>(gm));  // quad_perm [1,0,3,2]
    if (g >= 4) gm = fmaxf(gm, dpp_f<0x4E>(gm));  // quad_perm [2,3,0,1]
    const int ng = kThreads / g;
    if ((tid & (g - 1)) == 0) s_max[tid / g] = gm;
    if (tid == 0) s_lbk = key_of(kNegInf);
    __syncthreads();
    if (tid < ng) {
      const float mine = s_max[tid];
      int ge = 0;
#pragma unroll 2
      for (int j = 0; j < ng; j += 4) {
        const float4 t = *reinterpret_cast<const float4*>(&s_max[j]);
        ge += (t.x >= mine) + (t.y >= mine) + (t.z >= mine) + (t.w >= mine);
      }
      const float cand = (ge >= k && mine > kNegInf && mine < kPosInf) ? mine : kNegInf;
      const float wm = wave_max_dpp(cand);
      if ((tid & (kWave - 1)) == 0 && wm > kNegInf) atomicMax(&s_lbk, key_of(wm));
    }
    __syncthreads();
    lb = float_of_key(s_lbk);
  }
  const int flags = block_sum_i(bad) ? kRecFlagBad : 0;
  unsigned* rec = P.rec + (size_t)g * P.rec_words;
  unsigned* ent = rec + kRecHeader;
  // candidates: l >= lb, never -inf (an empty bound admits every finite logit)
  const float lb2 = (lb == kNegInf) ? -__FLT_MAX__ : lb;
  if (flags == 0 && k <= kBoundMaxK) {
    // No NaN or +inf here, so a vector holds a candidate iff its maximum
    // reaches the bound, and there are at most as many such vectors as
    // candidates. Stage them (thread order, then vector order) and count.
    __shared__ typename Vc::Raw s_hv[kHitMax];
    __shared__ int s_hid[kHitMax];
    unsigned hm = 0u;
#pragma unroll
    for (int u = 0; u < kFiltVpt; ++u) hm |= (vm[u] >= lb2 ? 1u : 0u) << u;
    int nhit;
    int hoff = block_excl_scan_i(__builtin_popcount(hm), nhit);
    if (nhit <= min(P.kcap, kHitMax)) {
#pragma unroll
      for (int u = 0; u < kFiltVpt; ++u) {
        if ((hm >> u) & 1u) {
          s_hv[hoff] = r[u];
          s_hid[hoff] = vb + u * kThreads + tid;
          ++hoff;
        }
      }
      __syncthreads();
      int cnt = 0;
      for (int j = tid; j < nhit; j += kThreads) {
        float f[N];
        Vc::get(s_hv[j], f);
#pragma unroll
        for (int k2 = 0; k2 < N; ++k2) cnt += (f[k2] >= lb2) ? 1 : 0;
      }
      int total;
      int off = block_excl_scan_i(cnt, total);
      if (total <= P.kcap) {
        for (int j = tid; j < nhit; j += kThreads) {
          float f[N];
          Vc::get(s_hv[j], f);
          const int id0 = s_hid[j] * N;
#pragma unroll
          for (int k2 = 0; k2 < N; ++k2) {
            if (f[k2] >= lb2) {
              ent[2 * off] = __float_as_uint(f[k2]);
              ent[2 * off + 1] = (unsigned)(id0 + k2);
              ++off;
            }
          }
        }
        if (tid == 0) {
          rec[0] = (unsigned)total;
          rec[1] = 0u;
          rec[2] = 0u;
          rec[3] = 0u;
          rec[4] = __float_as_uint(lb2);
        }
        return;
      }
    }
    // more candidates than the record holds: the exact cut below
  }
  int cnt = 0;
  each([&](float f, int) { cnt += (f >= lb2) ? 1 : 0; });
  int total;
  int off = block_excl_scan_i(cnt, total);
  if (total <= P.kcap) {
    each([&](float f, int id) {
      if (f >= lb2) {
        ent[2 * off] = __float_as_uint(f);
        ent[2 * off + 1] = (unsigned)id;
        ++off;
      }
    });
    if (tid == 0) {
      rec[0] = (unsigned)total;
      rec[1] = 0u;
      rec[2] = 0u;
      rec[3] = (unsigned)flags;
      rec[4] = __float_as_uint(lb2);
    }
    return;
  }
  // Exact k-th largest finite logit of the chunk, one key byte at a time from
  // the top (more than kcap > k candidates exist here).
  unsigned prefix = 0u, mask = 0u;
  int rem = k;
  for (int shift = 24; shift >= 0; shift -= 8) {
    s_hist[tid] = 0;
    __syncthreads();
    each([&](float f, int) {
      if (__builtin_isfinite(f) && f >= lb) {
        const unsigned key = key_of(f);
        if ((key & mask) == prefix) atomicAdd(&s_hist[(key >> shift) & 255u], 1);
      }
    });
    __syncthreads();
    select_bin(s_hist, rem, s_sel);
    __syncthreads();
    prefix |= (unsigned)s_sel[0] << shift;
    mask |= 255u << shift;
    rem = s_sel[1];
    __syncthreads();
  }
  const float tau = float_of_key(prefix);
  int gt = 0, eq = 0;
  each([&](float f, int) {
    if (__builtin_isfinite(f)) {
      gt += f > tau;
      eq += f == tau;
    }
  });
  const int gt_tot = block_sum_i(gt);
  const int eq_tot = block_sum_i(eq);
  const bool ties_fit = gt_tot + eq_tot <= P.kcap;  // gt_tot < k <= kcap always
  cnt = 0;
  each([&](float f, int) {
    cnt += (__builtin_isfinite(f) && (f > tau || (ties_fit && f == tau))) ? 1 : 0;
  });
  off = block_excl_scan_i(cnt, total);
  // (the bound holds for any row with at least k finite logits; the guard keeps
  // an invalid row, e.g. one full of +inf, inside its record)
  each([&](float f, int id) {
    if (__builtin_isfinite(f) && (f > tau || (ties_fit && f == tau)) && off < P.kcap) {
      ent[2 * off] = __float_as_uint(f);
      ent[2 * off + 1] = (unsigned)id;
      ++off;
    }
  });
  if (tid == 0) {
    rec[0] = (unsigned)min(total, P.kcap);
    rec[1] = __float_as_uint(tau);
    rec[2] = ties_fit ? 0u : (unsigned)eq_tot;
    rec[3] = (unsigned)(flags | (ties_fit ? 0 : kRecFlagImplicitTies));
    rec[4] = __float_as_uint(tau);
  }
}

}  // namespace

// Returns chunk records to zero (whole block): record r of `nrec`, at
// rec_of(r), loses its header and the entries the header counts. Groups of 16
// threads take one record each; a group reads the count before its stores.
template <class RecOf>
__device__ void zero_records(const Params& P, int nrec, RecOf rec_of) {
  constexpr int G = 16;
  const int grp = threadIdx.x / G, lane = threadIdx.x % G;
  for (int r = grp; r < nrec; r += kThreads / G) {
    unsigned* h = rec_of(r);
    if (h == nullptr) continue;
    const int words = kRecHeader + 2 * min((int)h[0], P.kcap);
    for (int w = lane; w < words; w += G) h[w] = 0u;
  }
}

// ---------------------------------------------------------------- stats unit
// Stats block g covers chunk g % chunks of unit g / chunks: draft row u for
// u < total_draft, else target row u - total_draft. Its partial goes to
// slots[g] (read after the kernel boundary).
template <int DT, bool VEC, bool FILT>
__device__ void stats_unit(const Params& P, long long g) {
  __shared__ int s_cu[kCuLds];
  const int unit = (int)(g / P.chunks);
  const int ch = (int)(g - (long long)unit * P.chunks);
  bool is_target;
  int row;
  row_of_unit(P, unit, is_target, row);
  bool greedy = P.all_greedy != 0;
  if (!greedy && P.greedy != nullptr) greedy = P.greedy[row_seq(P, row, is_target, s_cu)] != 0;
  if (greedy && !is_target) return;  // greedy sequences never read draft rows
  if (P.skip_bonus && is_target && is_bonus_row(P, row, s_cu)) return;
  const void* base = is_target ? P.target : P.draft;
  const size_t roff = (size_t)row * (size_t)P.V;
  const int vb = ch * P.chunk_vecs;
  const int ve = min(P.nvec, vb + P.chunk_vecs);
  unsigned long long packed;
  if constexpr (FILT) {
    if (!greedy) {
      topk_block<DT, VEC>(P, g, base, roff, ch);
      return;
    }
    packed = chunk_stats<DT, VEC, true>(P, base, roff, vb, ve, true);
  } else {
    packed = chunk_stats<DT, VEC>(P, base, roff, vb, ve, greedy);
  }
  if (threadIdx.x == 0) P.slots[g] = packed;
}

// The statistics pass (filtered calls, and rows too long for k_verify).
template <int DT, bool VEC, bool FILT>
__global__ __launch_bounds__(kThreads) void k_stats(const Params P) {
  stats_unit<DT, VEC, FILT>(P, (long long)blockIdx.x + P.stats_block0);
}

// ----------------------------------------------------------------- k_filter
// Per filtered sampling row: the row's k-th largest finite logit tau (tie
// classes counted with their multiplicity), the softmax masses 2^(l*c - R) of
// the levels at or above it, and the top-p cut: a level stays iff the mass of
// the strictly larger kept levels, over the top-k mass, is below top_p. The
// row keeps every id with l >= theta (the smallest kept level).
// Pages: aihero.vn "Speculative decoding", section "Cùng phân bố không có
// nghĩa cùng chuỗi mỗi lần" (the same temperature, top-k and top-p on both
// models' rows).
constexpr int kFiltBins = 2048;  // 11-bit key digits in the select

// The general path, one whole block per row: radix select over the chunk
// records, then the levels above tau sorted in descending order and cut. Its
// staging arrays live in `lds` (kFilterBlockWords words).
constexpr int kFilterPoolWords = kFiltBins > 2 * kFilterMaxLevels ? kFiltBins : 2 * kFilterMaxLevels;
constexpr int kFilterBlockWords = kFilterPoolWords + kFilterLdsKeys + 4 * kFilterLdsChunks +
                                  kFilterLdsChunks + 1;

template <int DT>
__device__ void filter_row_block(const Params& P, int unit, unsigned* lds) {
  // significant high bits of a logit's key: a widened bf16 or fp16 value
  // leaves the low 16 or 13 key bits constant (all zero for a positive value,
  // all one for a negative one), so two 11-bit digits fix its level
  constexpr int kPasses = DT == SV_F32 ? 3 : 2;
  constexpr int kLastShift = DT == SV_F32 ? 0 : 10;
  // One LDS pool serves, in turn, the select's histogram and the levels
  // (value, weight).
  unsigned* const s_pool = lds;
  int* const s_hist = reinterpret_cast<int*>(s_pool);
  float* const s_v = reinterpret_cast<float*>(s_pool);
  float* const s_w = s_v + kFilterMaxLevels;
  __shared__ int s_sel[2];
  __shared__ int s_n;
  unsigned* const s_key = lds + kFilterPoolWords;
  unsigned(*const s_hdr)[4] = reinterpret_cast<unsigned(*)[4]>(s_key + kFilterLdsKeys);
  int* const s_off = reinterpret_cast<int*>(s_key + kFilterLdsKeys + 4 * kFilterLdsChunks);
  const int tid = threadIdx.x;
  const bool is_target = unit >= P.total_draft;
  const int row = is_target ? unit - P.total_draft : unit;
  const int C = P.chunks;
  const unsigned* rec0 = P.rec + (size_t)unit * C * P.rec_words;
  // Stage the records in LDS when they fit: headers, then every entry's key.
  const bool hdr_staged = C <= kFilterLdsChunks;
  bool staged = hdr_staged;
  int E = 0;
  if (staged) {
    if (tid < C) {
      const unsigned* h = rec0 + (size_t)tid * P.rec_words;
      s_hdr[tid][0] = min(h[0], (unsigned)P.kcap);
      s_hdr[tid][1] = h[1];
      s_hdr[tid][2] = h[2];
      s_hdr[tid][3] = h[3];
    }
    __syncthreads();
    if (tid < kWave) {
      s_off[tid + 1] = wave_incl_scan_i(tid < C ? (int)s_hdr[tid][0] : 0);
      if (tid == 0) s_off[0] = 0;
    }
    __syncthreads();
    E = s_off[C];
    staged = E <= kFilterLdsKeys;
    if (staged) {
      for (int i0 = tid; i0 < E; i0 += 4 * kThreads) {
        unsigned val[4];
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const int i = i0 + j * kThreads;
          val[j] = 0u;
          if (i < E) {
            int lo = 0, hi = C - 1;  // chunk of entry i: the last with s_off <= i
            while (lo < hi) {
              const int mid = (lo + hi + 1) >> 1;
              if (s_off[mid] <= i) lo = mid;
              else hi = mid - 1;
            }
            val[j] = rec0[(size_t)lo * P.rec_words + kRecHeader + 2 * (i - s_off[lo])];
          }
        }
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const int i = i0 + j * kThreads;
          if (i < E) s_key[i] = key_of(__uint_as_float(val[j]));
        }
      }
      __syncthreads();
    }
  }
  // fn(key, multiplicity) over every explicit entry and implicit tie class,
  // spread over the block's threads
  auto for_entries = [&](auto&& fn) {
    if (staged) {
      for (int i = tid; i < E; i += kThreads) fn(s_key[i], 1);
      if (tid < C && (s_hdr[tid][3] & kRecFlagImplicitTies))
        fn(key_of(__uint_as_float(s_hdr[tid][1])), (int)s_hdr[tid][2]);
    } else {
      for (int ch = 0; ch < C; ++ch) {
        const unsigned* h = rec0 + (size_t)ch * P.rec_words;
        const int ne = min((int)h[0], P.kcap);
        for (int e = tid; e < ne; e += kThreads)
          fn(key_of(__uint_as_float(h[kRecHeader + 2 * e])), 1);
        if (tid == 0 && (h[3] & kRecFlagImplicitTies))
          fn(key_of(__uint_as_float(h[1])), (int)h[2]);
      }
    }
  };
  int n_fin = 0, bad = 0;
  for_entries([&](unsigned, int cnt) { n_fin += cnt; });
  for (int ch = tid; ch < C; ch += kThreads)
    bad |= (int)((hdr_staged ? s_hdr[ch][3] : rec0[(size_t)ch * P.rec_words + 3]) & kRecFlagBad);
  n_fin = block_sum_i(n_fin);
  bad = block_sum_i(bad);
  const int k = P.top_k;
  float tau = kNegInf;  // more than k finite logits: the k-th largest
  if (n_fin > k) {
    unsigned prefix = 0u, mask = 0u;
    int rem = k;
    for (int pass = 0; pass < kPasses; ++pass) {
      // digits: bits 31-21, 20-10, 9-0
      const int shift = pass == 0 ? 21 : (pass == 1 ? 10 : 0);
      const int width = pass == 2 ? 10 : 11;
      for (int b = tid; b < kFiltBins; b += kThreads) s_hist[b] = 0;
      __syncthreads();
      for_entries([&](unsigned key, int cnt) {
        if ((key & mask) == prefix)
          atomicAdd(&s_hist[(key >> shift) & ((1u << width) - 1u)], cnt);
      });
      __syncthreads();
      select_bin<kFiltBins>(s_hist, rem, s_sel);
      __syncthreads();
      prefix |= (unsigned)s_sel[0] << shift;
      mask |= ((1u << width) - 1u) << shift;
      rem = s_sel[1];
      __syncthreads();
    }
    // the key bits below the last digit, constant for this dtype
    if (kLastShift > 0) prefix |= (prefix & 0x80000000u) ? 0u : ((1u << kLastShift) - 1u);
    tau = float_of_key(prefix);
  }
  // levels above tau (fewer than k logits, at most a few tie classes), then tau
  if (tid == 0) s_n = 0;
  __syncthreads();
  int eq = 0;
  for_entries([&](unsigned key, int cnt) {
    const float v = float_of_key(key);
    if (v > tau) {
      const int at = atomicAdd(&s_n, 1);
      if (at < kFilterMaxLevels) {
        s_v[at] = v;
        s_w[at] = (float)cnt;
      }
    } else if (v == tau) {
      eq += cnt;
    }
  });
  eq = block_sum_i(eq);
  if (tid == 0 && eq > 0 && s_n < kFilterMaxLevels) {
    s_v[s_n] = tau;
    s_w[s_n] = (float)eq;
    ++s_n;
  }
  __syncthreads();
  const int n = min(s_n, kFilterMaxLevels);
  const float c = P.c;
  __shared__ float s_theta;
  if (n <= kWave) {
    // Few levels (the usual case): wave 0 sorts them in registers, then scans
    // their masses and cuts, with no block-wide steps.
    if (tid < kWave) {
      float v = tid < n ? s_v[tid] : kNegInf;
      float w = tid < n ? s_w[tid] : 0.0f;
      wave_sort_desc(v, w);
      const float m = n > 0 ? __shfl(v, 0) : kNegInf;
      const float R = ref_of(m, c);
      const float e = (tid < n) ? w * fast_exp2(fmaf(v, c, -R)) : 0.0f;
      const float incl = wave_incl_scan(e);
      const float S_k = __shfl(incl, kWave - 1);
      // top-p: the last level whose strictly-larger mass over S_k is below top_p
      int last = n - 1;
      if (P.top_p < 1.0f) {
        const unsigned long long ok = __ballot(tid < n && (incl - e) / S_k < P.top_p);
        last = ok ? 63 - __clzll(ok) : -1;
      }
      const float theta = (n > 0 && last >= 0) ? __shfl(v, last) : kPosInf;
      const float kincl = wave_incl_scan((tid < n && v >= theta) ? e : 0.0f);
      if (tid == kWave - 1) {
        P.rowres[unit] = RowRes{m, kincl, theta, bad ? 1 : 0};
        s_theta = theta;
      }
    }
  } else {
    int p2 = 2;
    while (p2 < n) p2 <<= 1;
    for (int x = n + tid; x < p2; x += kThreads) {
      s_v[x] = kNegInf;
      s_w[x] = 0.0f;
    }
    __syncthreads();
    // bitonic sort, descending by value
    for (int size = 2; size <= p2; size <<= 1) {
      for (int stride = size >> 1; stride > 0; stride >>= 1) {
        for (int x = tid; x < p2; x += kThreads) {
          const int y = x ^ stride;
          if (y > x) {
            const bool desc = (x & size) == 0;
            const float a = s_v[x], b = s_v[y];
            if (desc ? (a < b) : (a > b)) {
              s_v[x] = b;
              s_v[y] = a;
              const float t = s_w[x];
              s_w[x] = s_w[y];
              s_w[y] = t;
            }
          }
        }
        __syncthreads();
      }
    }
    const float m = n > 0 ? s_v[0] : kNegInf;
    const float R = ref_of(m, c);
    // masses in sorted order; each thread takes a contiguous run
    const int per = (p2 + kThreads - 1) / kThreads;
    const int x0 = min(tid * per, p2), x1 = min(x0 + per, p2);
    float local = 0.0f;
    for (int x = x0; x < x1; ++x) {
      const float w = (x < n) ? s_w[x] * fast_exp2(fmaf(s_v[x], c, -R)) : 0.0f;
      s_w[x] = w;
      local += w;
    }
    float S_k;
    const float incl = block_incl_scan(local, S_k);
    // top-p: the last entry whose strictly-larger mass over S_k is below top_p
    int last = n - 1;
    if (P.top_p < 1.0f) {
      float run = incl - local;
      int cand = -1;
      for (int x = x0; x < x1 && x < n; ++x) {
        if (run / S_k < P.top_p) cand = x;
        run += s_w[x];
      }
      last = block_max_i(cand);
    }
    const float theta = (n > 0 && last >= 0) ? s_v[last] : kPosInf;
    float kept = 0.0f;
    for (int x = x0; x < x1 && x < n; ++x)
      if (s_v[x] >= theta) kept += s_w[x];
    float S_f;
    block_incl_scan(kept, S_f);
    if (tid == 0) {
      P.rowres[unit] = RowRes{m, S_f, theta, bad ? 1 : 0};
      s_theta = theta;
    }
  }
  __syncthreads();
  const float theta = s_theta;
  if (is_target && !P.skip_bonus && P.kept != nullptr) {
    // A target row's kept set, listed for the final draw when every kept id
    // is an explicit entry (no count-only tie class at or above theta; none
    // when the caller keeps no lists).
    unsigned* kl = P.kept + (size_t)row * kKeptWords;
    __syncthreads();
    if (tid == 0) s_n = 0;
    __syncthreads();
    auto add = [&](float v, unsigned id) {
      const int at = atomicAdd(&s_n, 1);
      if (at < kExplicitMax) {
        kl[2 + 2 * at] = __float_as_uint(v);
        kl[3 + 2 * at] = id;
      }
    };
    int partial = 0;
    if (staged) {
      for (int i = tid; i < E; i += kThreads) {
        const float v = float_of_key(s_key[i]);
        if (v >= theta) {
          int lo = 0, hi = C - 1;  // chunk of entry i
          while (lo < hi) {
            const int mid = (lo + hi + 1) >> 1;
            if (s_off[mid] <= i) lo = mid;
            else hi = mid - 1;
          }
          add(v, rec0[(size_t)lo * P.rec_words + kRecHeader + 2 * (i - s_off[lo]) + 1]);
        }
      }
      if (tid < C && (s_hdr[tid][3] & kRecFlagImplicitTies) && __uint_as_float(s_hdr[tid][1]) >= theta)
        partial = 1;
    } else {
      for (int ch = 0; ch < C; ++ch) {
        const unsigned* h = rec0 + (size_t)ch * P.rec_words;
        const int ne = min((int)h[0], P.kcap);
        for (int e = tid; e < ne; e += kThreads) {
          const float v = __uint_as_float(h[kRecHeader + 2 * e]);
          if (v >= theta) add(v, h[kRecHeader + 2 * e + 1]);
        }
        if (tid == 0 && (h[3] & kRecFlagImplicitTies) && __uint_as_float(h[1]) >= theta) partial = 1;
      }
    }
    partial = block_sum_i(partial);
    if (tid == 0) {
      kl[0] = (unsigned)min(s_n, kExplicitMax);
      kl[1] = (partial || s_n > kExplicitMax) ? 1u : 0u;
    }
  }
  // Every row's records go back to zero (nothing reads them after this pass),
  // their lengths taken from the staged headers when there are some.
  __syncthreads();
  unsigned* recw = P.rec + (size_t)unit * C * P.rec_words;
  if (hdr_staged) {
    constexpr int G = 16;
    for (int ch = tid / G; ch < C; ch += kThreads / G) {
      const int words = kRecHeader + 2 * (int)s_hdr[ch][0];
      for (int w = tid % G; w < words; w += G) recw[(size_t)ch * P.rec_words + w] = 0u;
    }
  } else {
    zero_records(P, C, [&](int ch) { return recw + (size_t)ch * P.rec_words; });
  }
}

// The usual path, two waves per row, for bf16 and fp16 rows whose candidates
// fit: every chunk record's entries are loaded at once (the row's slots of 64
// entries of one chunk, split between the two waves), and the candidates at or
// above the row's bound (the largest chunk bound; the row's k-th largest is
// never below it) are counted in a histogram of 2048 bins of one level each,
// from the bound's level up. A widened bf16 or fp16 logit's low 16 or 13 key
// bits are constant, so a bin is one logit value and its count that value's
// multiplicity. The first wave then finds tau's bin (where the count from the
// top reaches k) and walks the bins from the top with their masses
// count * 2^(l*c - R) for the top-p cut; both waves list the kept set and
// return the records to zero. A row takes the general path instead (having
// written nothing) for fp32, more than 64 chunks or 32 slots, a chunk with NaN
// or +inf, at most k finite logits, or candidates beyond 2048 levels above the
// bound.
constexpr int kFiltRowsPerBlock = kThreads / (2 * kWave);
constexpr int kFastSlots = 32;                   // 64-entry slots of a row
constexpr int kHalfSlots = kFastSlots / 2;       // slots a wave holds
// Histogram words: bins in groups of 32 (one lane's), each group followed by
// four pad words, so a lane's group starts on 16 bytes and the groups of
// neighbouring lanes fall on different banks.
constexpr int kFastHistWords = kFiltBins + kFiltBins / 8;
__device__ __forceinline__ int fast_idx(int b) { return b + 4 * (b >> 5); }
enum { kFiltFast = 0, kFiltGeneral = 1, kFiltNone = 2 };

// Two rows per block: each row's two waves take the usual path together, then
// the whole block takes the rows that need the general path, one at a time, in
// the LDS the histograms held. Every wave passes every barrier.
template <int DT>
__global__ __launch_bounds__(kThreads) void k_filter(const Params P) {
  constexpr bool kFast = DT != SV_F32;
  constexpr int kLow = DT == SV_BF16 ? 16 : 13;
  constexpr unsigned kLowMask = (1u << kLow) - 1u;
  __shared__ __align__(16) unsigned s_fh[kFiltRowsPerBlock][kFastHistWords];
  __shared__ int s_state[kFiltRowsPerBlock], s_over[kFiltRowsPerBlock], s_kn[kFiltRowsPerBlock];
  __shared__ float s_theta[kFiltRowsPerBlock];
  static_assert(kFastHistWords >= kCuLds, "the first histogram holds the staged offsets");
  static_assert(kFiltRowsPerBlock * kFastHistWords >= kFilterBlockWords,
                "the histograms hold the general path's staging");
  int* const s_cu = reinterpret_cast<int*>(s_fh[0]);
  const int wave = threadIdx.x / kWave, lane = threadIdx.x & (kWave - 1);
  const int ri = wave >> 1, h = wave & 1;  // the row of this wave, and its half
  const long long units = (long long)P.total_draft + P.rows;
  const long long u = (long long)blockIdx.x * kFiltRowsPerBlock + ri;
  const bool valid = u < units;
  const int unit = valid ? (int)u : 0;
  bool is_target;
  int row;
  row_of_unit(P, unit, is_target, row);
  // greedy rows and skipped bonus rows have no records (whole block: the
  // offsets are staged once per call)
  bool skip = !valid;
  if (P.greedy != nullptr) skip |= P.greedy[row_seq(P, row, is_target, s_cu)] != 0;
  if (P.skip_bonus) {
    const bool bonus = is_bonus_row(P, is_target ? row : 0, s_cu);
    skip |= is_target && bonus;
  }
  if (threadIdx.x < kFiltRowsPerBlock) {
    s_over[threadIdx.x] = 0;
    s_kn[threadIdx.x] = 0;
  }
  __syncthreads();  // the staged offsets are read before the histograms reuse them
  unsigned* const hist = s_fh[ri];
  const int C = P.chunks;
  const unsigned* rec0 = P.rec + (size_t)unit * C * P.rec_words;
  // chunk c's header in lane c: entries, tie value, tie count, flags; bound
  bool ok = kFast && !skip && C <= kWave;
  uint4 hd = make_uint4(0u, 0u, 0u, 0u);
  unsigned hb = 0u;
  if (ok && lane < C) {
    const unsigned* hp = rec0 + (size_t)lane * P.rec_words;
    hd = *reinterpret_cast<const uint4*>(hp);
    hb = hp[4];
  }
  const int cnt = lane < C ? min((int)hd.x, P.kcap) : 0;
  const bool imp = lane < C && (hd.w & kRecFlagImplicitTies) != 0u;
  int nq = 0, qexcl = 0, nslots = 0, soff = 0, slim = 0;
  float bnd = kNegInf;
  unsigned kb = 0u;
  if (ok) {  // wave-uniform; both waves of a row reach the same decisions
    ok = __builtin_amdgcn_ballot_w64(lane < C && (hd.w & kRecFlagBad) != 0u) == 0ull;
    nq = (cnt + kWave - 1) / kWave;  // slots of chunk `lane`
    qexcl = wave_incl_scan_i(nq) - nq;
    nslots = __builtin_amdgcn_readlane(qexcl + nq, kWave - 1);
    ok = ok && nslots <= kFastSlots;
    ok = ok && wave_sum_i(cnt + (imp ? (int)hd.z : 0)) > P.top_k;
    bnd = wave_max_dpp(lane < C ? __uint_as_float(hb) : kNegInf);
    ok = ok && bnd > -__FLT_MAX__;
    kb = key_of(bnd) & ~kLowMask;  // bin 0: the bound's level
    // Slot table in lanes 0..31: slot s holds entries 64*(s - first slot of
    // its chunk) + lane of chunk c(s), the last chunk whose first slot is at or
    // before s. soff: the word offset of the slot's first entry; slim: its
    // number of entries.
    int cs = 0;
    for (int cc = 1; cc < C; ++cc) cs += (__builtin_amdgcn_readlane(qexcl, cc) <= lane) ? 1 : 0;
    const int e0 = (lane - __shfl(qexcl, cs)) * kWave;
    soff = cs * P.rec_words + kRecHeader + 2 * e0;
    slim = lane < nslots ? min(kWave, __shfl(cnt, cs) - e0) : 0;
  }
  // This wave's slots h, h + 2, ...: every one is loaded, with no branch, so
  // that all the loads are in flight together. A slot past the last reads the
  // first slot's entries, and a lane past its slot's count reads a zero entry
  // of the same record (a slot never runs past its chunk's kcap entries).
  // vmask marks the entries.
  uint2 ev[kHalfSlots];
  unsigned vmask = 0u;
  if (ok) {
#pragma unroll
    for (int j = 0; j < kHalfSlots; ++j) {
      const int s = 2 * j + h;
      const int so = s < nslots ? __builtin_amdgcn_readlane(soff, s) : __builtin_amdgcn_readlane(soff, 0);
      ev[j] = *reinterpret_cast<const uint2*>(rec0 + so + 2 * lane);
      if (s < nslots && lane < __builtin_amdgcn_readlane(slim, s)) vmask |= 1u << j;
    }
    for (int i = h * kWave + lane; i < kFastHistWords / 4; i += 2 * kWave)
      reinterpret_cast<uint4*>(hist)[i] = make_uint4(0u, 0u, 0u, 0u);
  }
  __syncthreads();  // the histograms are clear
  if (ok) {
    // count the candidates at or above the bound by level; a candidate beyond
    // the last bin goes to the last pad word and makes the row take the
    // general path
    bool over = false;
    auto add = [&](float v, unsigned n) {
      const unsigned bin = (key_of(v) - kb) >> kLow;
      over |= bin >= (unsigned)kFiltBins;
      atomicAdd(&hist[bin < (unsigned)kFiltBins ? fast_idx((int)bin) : kFastHistWords - 1], n);
    };
#pragma unroll
    for (int j = 0; j < kHalfSlots; ++j) {
      const float v = __uint_as_float(ev[j].x);
      if (((vmask >> j) & 1u) && v >= bnd) add(v, 1u);
    }
    if (h == 0 && imp && __uint_as_float(hd.y) >= bnd) add(__uint_as_float(hd.y), hd.z);
    if (__builtin_amdgcn_ballot_w64(over) != 0ull && lane == 0) s_over[ri] = 1;
  }
  __syncthreads();  // the counts and the overflow marks are in
  ok = ok && s_over[ri] == 0;
  if (h == 0) {
    int state = skip ? kFiltNone : kFiltGeneral;
    if (ok) {
      // lane l holds the 32 bins of group 63 - l (lane 0 the top ones); bit j
      // of nzm: bin top - j is not empty
      const int g = kWave - 1 - lane;
      const int top = 32 * g + 31;
      const uint4* hg = reinterpret_cast<const uint4*>(hist + 36 * g);
      int lsum = 0;
      unsigned nzm = 0u;
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const uint4 q = hg[i];  // bins 32g + 4i .. 32g + 4i + 3, that is j = 31 - 4i - t
        lsum += (int)(q.x + q.y + q.z + q.w);
        nzm |= ((q.x != 0u) ? 1u : 0u) << (31 - 4 * i) | ((q.y != 0u) ? 1u : 0u) << (30 - 4 * i) |
               ((q.z != 0u) ? 1u : 0u) << (29 - 4 * i) | ((q.w != 0u) ? 1u : 0u) << (28 - 4 * i);
      }
      // tau: the bin where the count from the top reaches k (lane ft's group,
      // then its bins, one per lane)
      const int k = P.top_k;
      const int incl = wave_incl_scan_i(lsum);
      const unsigned long long hit = __builtin_amdgcn_ballot_w64(incl >= k);
      const int ft = hit ? __ffsll((unsigned long long)hit) - 1 : 0;
      const int above_ft = __builtin_amdgcn_readlane(incl - lsum, ft);
      const int top_ft = 32 * (kWave - 1 - ft) + 31;
      const int cj = lane < 32 ? (int)hist[fast_idx(top_ft - lane)] : 0;
      const unsigned long long hit2 =
          __builtin_amdgcn_ballot_w64(lane < 32 && above_ft + wave_incl_scan_i(cj) >= k);
      const int btau = top_ft - (hit2 ? __ffsll((unsigned long long)hit2) - 1 : 0);
      // the row maximum: the top non-empty bin
      const int fm = __ffsll((unsigned long long)__builtin_amdgcn_ballot_w64(nzm != 0u)) - 1;
      const int bmax =
          32 * (kWave - 1 - fm) + 31 - (__ffs((int)__builtin_amdgcn_readlane((int)nzm, fm)) - 1);
      auto level = [&](int b) {
        unsigned key = kb + ((unsigned)b << kLow);
        if (!(key & 0x80000000u)) key |= kLowMask;
        return float_of_key(key);
      };
      const float c = P.c;
      const float m = level(bmax);
      const float R = ref_of(m, c);
      // the levels from tau up: this lane's non-empty bins at or above btau,
      // in descending order; their masses replace their counts
      const unsigned ftmask = 0xFFFFFFFFu >> (31 - (top_ft - btau));  // lane ft's bins down to btau
      const unsigned live = lane < ft ? nzm : (lane == ft ? nzm & ftmask : 0u);
      float esum = 0.0f;
      for (unsigned mm = live; mm != 0u; mm &= mm - 1u) {
        const int b = top - (__ffs((int)mm) - 1);
        unsigned* hw = &hist[fast_idx(b)];
        const float e = (float)*hw * fast_exp2(fmaf(level(b), c, -R));
        *hw = __float_as_uint(e);
        esum += e;
      }
      const float eincl = wave_incl_scan(esum);
      const float S_k = __builtin_bit_cast(float, __builtin_amdgcn_readlane(
                                                      __builtin_bit_cast(int, eincl), kWave - 1));
      // kept: the mass of the strictly larger levels over S_k below top_p
      // (every level from tau up when top_p is 1)
      const bool all = !(P.top_p < 1.0f);
      float above = eincl - esum, kincl = 0.0f;
      int bk = -1;
      for (unsigned mm = live; mm != 0u; mm &= mm - 1u) {
        const int b = top - (__ffs((int)mm) - 1);
        const float e = __uint_as_float(hist[fast_idx(b)]);
        if (all || above / S_k < P.top_p) {
          bk = b;
          kincl = above + e;
        }
        above += e;
      }
      const unsigned long long kept_lanes = __builtin_amdgcn_ballot_w64(bk >= 0);
      if (hit != 0ull && hit2 != 0ull && kept_lanes != 0ull) {
        const int lk = 63 - __clzll((long long)kept_lanes);
        const float theta = level(__builtin_amdgcn_readlane(bk, lk));
        const float S_f = __builtin_bit_cast(float, __builtin_amdgcn_readlane(
                                                        __builtin_bit_cast(int, kincl), lk));
        if (lane == 0) {
          P.rowres[unit] = RowRes{m, S_f, theta, 0};
          s_theta[ri] = theta;
        }
        state = kFiltFast;
      }
    }
    if (lane == 0) s_state[ri] = state;
  }
  __syncthreads();  // every row's state and theta are in
  const int state = s_state[ri];
  const bool lists = is_target && !P.skip_bonus && P.kept != nullptr;
  bool partial = false;
  if (state == kFiltFast) {
    const float theta = s_theta[ri];
    if (lists) {
      // the kept set (no count-only tie class at or above theta): each slot's
      // kept entries take consecutive places of the list
      unsigned* kl = P.kept + (size_t)row * kKeptWords;
#pragma unroll
      for (int j = 0; j < kHalfSlots; ++j) {
        const bool in = ((vmask >> j) & 1u) && __uint_as_float(ev[j].x) >= theta;
        const unsigned long long msk = __builtin_amdgcn_ballot_w64(in);
        if (msk != 0ull) {
          int base = 0;
          if (lane == 0) base = atomicAdd(&s_kn[ri], __builtin_popcountll(msk));
          base = __builtin_amdgcn_readfirstlane(base);
          const int at = base + (int)__builtin_amdgcn_mbcnt_hi(
                                    (unsigned)(msk >> 32), __builtin_amdgcn_mbcnt_lo((unsigned)msk, 0u));
          if (in && at < kExplicitMax) *reinterpret_cast<uint2*>(kl + 2 + 2 * at) = ev[j];
        }
      }
      partial = h == 0 &&
                __builtin_amdgcn_ballot_w64(imp && __uint_as_float(hd.y) >= theta) != 0ull;
    }
    // the records go back to zero: every slot's span (entries past a chunk's
    // count are zero already), then the headers
    unsigned* recw = P.rec + (size_t)unit * C * P.rec_words;
#pragma unroll
    for (int j = 0; j < kHalfSlots; ++j) {
      const int s = 2 * j + h;
      if (s < nslots)
        *reinterpret_cast<uint2*>(recw + __builtin_amdgcn_readlane(soff, s) + 2 * lane) =
            make_uint2(0u, 0u);
    }
    if (h == 0 && lane < C) {
      uint4* hp = reinterpret_cast<uint4*>(recw + (size_t)lane * P.rec_words);
      hp[0] = make_uint4(0u, 0u, 0u, 0u);
      hp[1] = make_uint4(0u, 0u, 0u, 0u);
    }
  }
  __syncthreads();  // the kept counts are in
  if (state == kFiltFast && lists && h == 0 && lane == 0) {
    unsigned* kl = P.kept + (size_t)row * kKeptWords;
    const int n = s_kn[ri];
    kl[0] = (unsigned)min(n, kExplicitMax);
    kl[1] = (partial || n > kExplicitMax) ? 1u : 0u;
  }
  for (int w = 0; w < kFiltRowsPerBlock; ++w) {
    if (s_state[w] == kFiltGeneral) {
      __syncthreads();  // the LDS of the histograms, or of the previous row, is free
      filter_row_block<DT>(P, blockIdx.x * kFiltRowsPerBlock + w, &s_fh[0][0]);
    }
  }
}

// ---------------------------------------------------------------- k_nucleus
// One block per sampling row when top-p acts without top-k: the row's
// threshold theta (keep l >= theta) and the kept-set sum, found by a radix
// descent on order-preserving keys. Each pass adds the mass 2^(l*c - R) of
// every logit whose key lies in the range fixed so far, in 40-bit fixed point
// (integer sums: exact and independent of the order of addition), to the bin
// of its key. Walking the bins from the largest key down, the kept levels are
// those whose strictly-larger mass is below top_p times the row total S (the
// sum the statistics pass formed, merged here in chunk order); the last of
// them lies in the bin where the running mass, this bin included, first
// reaches that bound, and the next pass splits that bin. The first pass bins
// only the keys of the top window (masses from 2^-16 of the maximum's up), in
// at most 2048 equal bins no narrower than one level (a widened bf16 or fp16
// logit's low 16 or 13 key bits are constant). A logit below the window costs
// one compare with the window's lowest value; the mass, its fixed point and
// the LDS add are spent on the window's logits alone (about 2% of a row at
// the sampling workloads). When the level lies in the window (the usual case)
// and the window holds at most 2048 levels (a bf16 row at the temperatures of
// sampling), one pass resolves it. Otherwise a pass bins the keys below the
// window down to the 2^-40 cutoff, and each further pass divides the bin by
// 2^11, so an fp32 level takes at most four. The row's chunk partials (read
// here only) go back to zero.
// Pages: aihero.vn "Speculative decoding", section "Cùng phân bố không có
// nghĩa cùng chuỗi mỗi lần" (the same temperature, top-k and top-p on both
// models' rows).
constexpr int kNucBins = 2048;
// The first pass bins only the logits within 2^-16 of the row maximum's mass
// (the top window): at the sampling workloads it holds about 2% of a row's
// logits and over 98% of its mass, so the top-p level nearly always lies in
// it, and the rest of the row only adds to the total.
constexpr double kNucScale = 1099511627776.0;  // 2^40
constexpr float kNucTop = 16.0f;
constexpr int kNucRing = 128;  // candidates a wave holds in LDS: twice a wave
#ifndef SV_NUC_THREADS
#define SV_NUC_THREADS 256
#endif
// Threads of a k_nucleus block (one block per row). The bin scan runs on the
// first kNucScan of them.
constexpr int kNucThreads = SV_NUC_THREADS;
constexpr int kNucScan = 256;
static_assert(kNucThreads % kWave == 0 && kNucThreads >= kNucScan && kNucBins % kNucScan == 0,
              "whole waves, and the scan's threads take equal runs of bins");

template <int DT, bool VEC>
__global__ __launch_bounds__(kNucThreads) void k_nucleus(const Params P) {
  using Vc = Vec<DT, VEC>;
  constexpr int N = Vc::N;
  __shared__ unsigned long long s_hist[kNucBins];
  __shared__ unsigned long long s_wave[kNucScan / kWave];
  __shared__ unsigned long long s_base;
  __shared__ int s_cu[kCuLds];
  __shared__ float s_stat[2];
  __shared__ unsigned s_kmin[2];
  __shared__ int s_bin;
  __shared__ float s_ring[kNucThreads / kWave][kNucRing];
  const int tid = threadIdx.x;
  const int lane = tid & (kWave - 1);
  const int unit = blockIdx.x;
  const bool is_target = unit >= P.total_draft;
  const int row = is_target ? unit - P.total_draft : unit;
  if (P.greedy != nullptr && P.greedy[row_seq(P, row, is_target, s_cu)] != 0) return;
  if (P.skip_bonus && is_target && is_bonus_row(P, row, s_cu)) return;
  const int C = P.chunks;
  const float c = P.c;
  unsigned long long* sl = P.slots + (size_t)unit * C;
  if (tid == 0) {
    float m = kNegInf, sm = 0.f;
    for (int k = 0; k < C; ++k) {
      float om, os;
      unpack_ms(sl[k], om, os);
      merge_ms(m, sm, om, os, c);
    }
    s_stat[0] = m;
    s_stat[1] = sm;
  }
  __syncthreads();
  if (tid < 2 * kWave) {
    // The smallest keys whose logits pass the mass tests below (2^-40 by wave
    // 0, the top window's 2^-kNucTop by wave 1): each test is monotone in the
    // key, fails at -inf and holds at the maximum. Each round the wave probes
    // 64 keys spread over (lo, hi]; the passing probes are a suffix of the
    // lanes, and the first of them and the one before it bound the key anew,
    // so the interval shrinks 64-fold a round and the key is found exactly.
    const float m0 = s_stat[0];
    const float cut = tid < kWave ? -40.0f : -kNucTop;
    unsigned lo = key_of(kNegInf), hi = lo;
    if (__builtin_isfinite(m0)) {
      const float R0 = ref_of(m0, c);
      hi = key_of(m0);
      while (hi - lo > 1u) {
        const unsigned long long span = hi - lo;
        const unsigned probe =
            lo + (unsigned)((span * (unsigned long long)(lane + 1) + kWave - 1) / kWave);
        const bool pass = fmaf(float_of_key(probe), c, -R0) >= cut;
        // lane 63 probes hi, which passes
        const int first = __ffsll((unsigned long long)__builtin_amdgcn_ballot_w64(pass)) - 1;
        const unsigned below = __shfl(probe, first > 0 ? first - 1 : 0);
        hi = __shfl(probe, first);
        lo = first > 0 ? below : lo;
      }
    }
    if (lane == 0) s_kmin[tid / kWave] = hi;
  }
  __syncthreads();
  for (int k = tid; k < C; k += kNucThreads) sl[k] = 0ull;
  const float m = s_stat[0];
  const bool ok = __builtin_isfinite(m) && s_stat[1] > 0.f && __builtin_isfinite(s_stat[1]);
  const float R = ref_of(m, c);
  const size_t roff = (size_t)row * P.V;
  const void* base = is_target ? P.target : P.draft;
  // low key bits every level of the input type shares
  constexpr int kLowBits = DT == SV_BF16 ? 16 : (DT == SV_F16 ? 13 : 0);
  constexpr unsigned kLowMask = (1u << kLowBits) - 1u;
  // The first pass bins the keys [kbase, kbase + span] of the top window
  // (from the smallest key passing its test, widened to a level boundary, to
  // the maximum's). When the crossing lies below the window, the next pass
  // bins the keys below it that can carry mass.
  // Each pass covers the keys [kbase, kbase + span], never above kmax: the
  // maximum's key in the window, kb_top - 1 below it (the window's mass is
  // already counted as the mass above), so a split bin never reaches back
  // into a range another pass has summed.
  const unsigned kb_all = s_kmin[0] & ~kLowMask, kb_top = s_kmin[1] & ~kLowMask;
  unsigned kbase = 0u, span = 0u, kmax = 0u;
  int s = kLowBits;
  if (ok) {
    kbase = kb_top;
    kmax = key_of(m);
    span = kmax - kbase;
  }
  bool found = false;  // a level has been resolved (else every level is kept)
  unsigned long long above = 0ull, kept = 0ull;
  const double bound = (double)P.top_p * (double)s_stat[1] * kNucScale;
  const int nb = kNucBins;
  // the wave's index, known to the compiler as wave-uniform (scalar loop bounds)
  const int wv = __builtin_amdgcn_readfirstlane(tid / kWave);
  float* ring = s_ring[wv];
  for (int lv = 0; ok; ++lv) {
    // bins of 2^s keys: the fewest that leave at most nb of them
    s = kLowBits;
    while ((span >> s) >= (unsigned)nb) ++s;
    for (int x = tid; x < nb; x += kNucThreads) s_hist[x] = 0ull;
    __syncthreads();
    // A logit of the pass's key range: its mass in fixed point, into the bin
    // of its key. Keys below the range wrap past span. A mass below 2^-40
    // (possible only at the level-widened low end of the range) adds zero.
    auto add = [&](float l) {
      const unsigned d = key_of(l) - kbase;
      if (d > span) return;
      const unsigned long long q =
          (unsigned long long)(fast_exp2(fmaf(l, c, -R)) * (float)kNucScale);
      atomicAdd(&s_hist[d >> s], q);
    };
    // The candidates of each wave (a superset of the range: lo_f <= l <= hi_f,
    // which NaN fails) are appended to the wave's ring in LDS in ballot order,
    // and the wave adds them 64 at a time with every lane busy: about 2% of
    // the logits pass in the window pass, so adding them where they were
    // loaded would run the add for one or two lanes at a time. n and head
    // count appended and added candidates; both are wave-uniform, so every
    // loop below runs on wave-uniform bounds.
    const float lo_f = float_of_key(kbase), hi_f = float_of_key(kbase + span);
    unsigned n = 0u, head = 0u;
    auto drain64 = [&]() {
      __builtin_amdgcn_wave_barrier();
      add(ring[(head + lane) & (kNucRing - 1)]);
      head += kWave;
      __builtin_amdgcn_wave_barrier();
    };
    // The window pass skips the upper test: no logit lies above the maximum.
    auto stage = [&](float l, auto upper) {
      const bool in = decltype(upper)::value ? (l >= lo_f && l <= hi_f) : (l >= lo_f);
      const unsigned long long msk = __builtin_amdgcn_ballot_w64(in);
      if (msk == 0ull) return;
      if (in) {
        const unsigned pos = __builtin_amdgcn_mbcnt_hi(
            (unsigned)(msk >> 32), __builtin_amdgcn_mbcnt_lo((unsigned)msk, n));
        ring[pos & (kNucRing - 1)] = l;
      }
      n += (unsigned)__popcll(msk);
      // fewer than 64 were pending before this append, so the ring of 128
      // never overwrites one not yet added
      if (n - head >= (unsigned)kWave) drain64();
    };
    // The row is streamed with non-temporal loads, as in the statistics pass
    // (measured 60 against 64 us with ordinary loads at the headline shape).
    auto stream = [&](auto upper) {
      int vb = wv * kWave;  // the wave's first vector
      for (; vb + kWave - 1 + (kBatch - 1) * kNucThreads < P.nvec; vb += kBatch * kNucThreads) {
        typename Vc::Raw r[kBatch];
#pragma unroll
        for (int u = 0; u < kBatch; ++u)
          r[u] = Vc::load_stream(base, roff, vb + lane + u * kNucThreads);
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int u = 0; u < kBatch; ++u) {
          float f[N];
          Vc::get(r[u], f);
#pragma unroll
          for (int k = 0; k < N; ++k) stage(f[k], upper);
        }
      }
      for (; vb < P.nvec; vb += kNucThreads) {
        const int v = vb + lane;
        float f[N];
        if (v < P.nvec) {
          Vc::get(Vc::load_stream(base, roff, v), f);
        } else {
#pragma unroll
          for (int k = 0; k < N; ++k) f[k] = __builtin_nanf("");
        }
#pragma unroll
        for (int k = 0; k < N; ++k) stage(f[k], upper);
      }
    };
    if (lv == 0) stream(std::false_type{});
    else stream(std::true_type{});
    __builtin_amdgcn_wave_barrier();
    if (lane < (int)(n - head)) add(ring[(head + lane) & (kNucRing - 1)]);
    __syncthreads();
    // scan thread t sums a run of bins in descending key order, then an
    // exclusive scan over those threads gives the mass above each run
    const bool scanner = tid < kNucScan;
    const int per = nb / kNucScan;
    const int top = nb - 1 - tid * per;
    unsigned long long run = 0ull, incl = 0ull;
    if (scanner) {
      for (int k = 0; k < per; ++k) run += s_hist[top - k];
      incl = run;
#pragma unroll
      for (int o = 1; o < kWave; o <<= 1) {
        const unsigned long long y = __shfl_up(incl, o);
        if (lane >= o) incl += y;
      }
      if (lane == kWave - 1) s_wave[tid / kWave] = incl;
    }
    if (tid == 0) s_bin = -1;
    __syncthreads();
    unsigned long long before = 0ull, total = 0ull;
    for (int w = 0; w < kNucScan / kWave; ++w) {
      if (w < tid / kWave) before += s_wave[w];
      total += s_wave[w];
    }
    if (scanner) {
      unsigned long long acc = above + before + (incl - run);
      for (int k = 0; k < per; ++k) {
        const unsigned long long h = s_hist[top - k];
        // the strictly-larger mass acc is below the bound and the running mass
        // reaches it in this bin: the last kept level lies here
        if ((double)acc < bound && (double)(acc + h) >= bound) {
          s_bin = top - k;
          s_base = acc;
        }
        acc += h;
      }
    }
    __syncthreads();
    if (s_bin < 0) {
      if (lv == 0 && kb_top > kb_all) {
        // below the top window: its mass is strictly larger than every level left
        above += total;
        kbase = kb_all;
        kmax = kb_top - 1u;
        span = kmax - kbase;
        continue;
      }
      break;  // the bound lies past every level: all are kept
    }
    found = true;
    kbase += (unsigned)s_bin << s;
    above = s_base;
    kept = s_base + s_hist[s_bin];
    __syncthreads();
    if (s == kLowBits) break;  // the bin is one level
    span = min((1u << s) - 1u, kmax - kbase);
  }
  if (tid == 0) {
    RowRes rr;
    rr.m = m;
    rr.flags = ok ? 0 : 1;
    if (!ok || !found) {
      rr.theta = kNegInf;  // every level kept
      rr.s = s_stat[1];
    } else {
      // the level's constant low key bits: zero for a positive value, ones
      // for a negative one (its key is the complement of its bits)
      const unsigned key = kbase | ((kbase & 0x80000000u) ? 0u : kLowMask);
      rr.theta = float_of_key(key);
      rr.s = (float)((double)kept / kNucScale);
    }
    P.rowres[unit] = rr;
  }
}

// Returns the partials of a sequence's rows to zero (whole block): its target
// rows and, with_draft, its draft rows.
__device__ void clear_partials(const Params& P, int d0, int kb, int b, bool with_draft) {
  const int C = P.chunks;
  const int nd = with_draft ? kb : 0;
  for (int k = threadIdx.x; k < (nd + kb + 1) * C; k += kThreads) {
    const int r = k / C, ch = k - r * C;
    const bool tgt = r >= nd;
    pub_u64(P.slots + unit_of(P, tgt, tgt ? d0 + b + (r - nd) : d0 + r) * C + ch, 0ull);
  }
}

// Final draw of a filtered sequence from the kept list of row p_n (whole
// block): p_n is zero outside its kept set, which the filter pass lists in
// full unless a tie class at the cut was kept as a count or the set exceeds
// kExplicitMax ids. The residual max(0, p_n - q_n) (or p_n for the bonus) is
// formed on those ids alone, with q_n's logit loaded at each id; the weights
// are sorted by id and scanned for the first cumulative weight above u*Z, as
// the inverse CDF over the whole row would. explicit_usable is false (in every
// thread) when the list is not complete; the caller then draws from the rows.
__device__ bool explicit_usable(const Params& P, const Job& j) {
  return P.kept[(size_t)j.prow * kKeptWords + 1] == 0u;
}

template <int DT>
__device__ int explicit_draw(const Params& P, const Job& j, float& Zout) {
  __shared__ int s_id[kExplicitMax];
  __shared__ float s_lp[kExplicitMax];
  __shared__ float s_wt[kExplicitMax];
  __shared__ int s_cnt;
  const int tid = threadIdx.x;
  const float c = P.c;
  const unsigned* kl = P.kept + (size_t)j.prow * kKeptWords;
  if ((int)kl[0] <= kWave) {
    // Few kept ids (the usual case): wave 0 reads the count and the first 64
    // entries in one round (words past the count read zero), then sorts,
    // scans and picks in registers.
    __shared__ int s_tok;
    __shared__ float s_Z;
    if (tid < kWave) {
      const int n = (int)kl[0];
      const unsigned lv = kl[2 + 2 * tid], li = kl[3 + 2 * tid];
      const bool in = tid < n;
      int id = in ? (int)li : INT_MAX;
      float lp = in ? __uint_as_float(lv) : kNegInf;
      float w = 0.0f;
      if (in) {
        const float ep = fast_exp2(fmaf(lp, c, -j.Rp));
        if (j.mode == kJobBonus) {
          w = ep * j.invSp;
        } else {
          const float lq = load_elem<DT>(P.draft, (size_t)j.qrow * P.V + id);
          const float q = (lq >= j.thr_q) ? fast_exp2(fmaf(lq, c, -j.Rq)) * j.invSq : 0.0f;
          w = fmaxf(fmaf(ep, j.invSp, -q), 0.0f);
        }
      }
      wave_sort_by_id(id, w, lp);
      float incl = wave_incl_scan(w);
      float total = __shfl(incl, kWave - 1);
      if (!(total > 0.0f) && j.mode == kJobResidual) {
        // the residual mass rounded to zero: draw from p_n instead
        w = (id != INT_MAX) ? fast_exp2(fmaf(lp, c, -j.Rp)) * j.invSp : 0.0f;
        incl = wave_incl_scan(w);
        total = __shfl(incl, kWave - 1);
      }
      const float target = j.u * total;
      const float excl = incl - w;
      const unsigned long long hit = __ballot(excl + w > target);
      const unsigned long long pos = __ballot(w > 0.0f);
      const int at = hit ? __ffsll(hit) - 1 : (pos ? 63 - __clzll(pos) : -1);
      const int tok_at = __shfl(id, at >= 0 ? at : 0);
      if (tid == 0) {
        s_tok = (at >= 0 && at < n) ? tok_at : id;
        s_Z = total;
      }
    }
    __syncthreads();
    Zout = s_Z;
    return s_tok;
  }
  if (tid == 0) s_cnt = (int)kl[0];
  __syncthreads();
  for (int x = tid; x < s_cnt; x += kThreads) {
    s_lp[x] = __uint_as_float(kl[2 + 2 * x]);
    s_id[x] = (int)kl[3 + 2 * x];
  }
  __syncthreads();
  const int n = min(s_cnt, kExplicitMax);
  int p2 = 2;
  while (p2 < n) p2 <<= 1;
  // weights; pads sort last with zero weight
  for (int x = tid; x < p2; x += kThreads) {
    if (x < n) {
      const float ep = fast_exp2(fmaf(s_lp[x], c, -j.Rp));
      float w;
      if (j.mode == kJobBonus) {
        w = ep * j.invSp;
      } else {
        const float lq = load_elem<DT>(P.draft, (size_t)j.qrow * P.V + s_id[x]);
        const float q = (lq >= j.thr_q) ? fast_exp2(fmaf(lq, c, -j.Rq)) * j.invSq : 0.0f;
        w = fmaxf(fmaf(ep, j.invSp, -q), 0.0f);
      }
      s_wt[x] = w;
    } else {
      s_id[x] = INT_MAX;
      s_lp[x] = kNegInf;
      s_wt[x] = 0.0f;
    }
  }
  __syncthreads();
  // bitonic sort by id, ascending
  for (int size = 2; size <= p2; size <<= 1) {
    for (int stride = size >> 1; stride > 0; stride >>= 1) {
      for (int x = tid; x < p2; x += kThreads) {
        const int y = x ^ stride;
        if (y > x) {
          const bool up = (x & size) == 0;
          const int a = s_id[x], bb = s_id[y];
          if (up ? (a > bb) : (a < bb)) {
            s_id[x] = bb;
            s_id[y] = a;
            const float t = s_wt[x];
            s_wt[x] = s_wt[y];
            s_wt[y] = t;
            const float tl = s_lp[x];
            s_lp[x] = s_lp[y];
            s_lp[y] = tl;
          }
        }
      }
      __syncthreads();
    }
  }
  // inclusive scan in id order (each thread a contiguous run), then the pick
  const int per = (p2 + kThreads - 1) / kThreads;
  const int x0 = min(tid * per, p2), x1 = min(x0 + per, p2);
  int tok = INT_MAX;
  float Z = 0.0f;
  for (int pass = 0; pass < 2; ++pass) {
    float local = 0.0f;
    for (int x = x0; x < x1; ++x) local += s_wt[x];
    float total;
    const float incl = block_incl_scan(local, total);
    if (pass == 0 && !(total > 0.0f) && j.mode == kJobResidual) {
      // the residual mass rounded to zero: draw from p_n instead
      for (int x = x0; x < x1; ++x)
        s_wt[x] = (x < n) ? fast_exp2(fmaf(s_lp[x], c, -j.Rp)) * j.invSp : 0.0f;
      __syncthreads();
      continue;
    }
    Z = total;
    const float target = j.u * total;
    float run = incl - local;
    int cand = INT_MAX, lastpos = -1;
    for (int x = x0; x < x1; ++x) {
      const float w = s_wt[x];
      if (cand == INT_MAX && run + w > target) cand = x;
      if (w > 0.0f) lastpos = x;
      run += w;
    }
    int at = block_min_i(cand);
    if (at == INT_MAX) at = block_max_i(lastpos);
    tok = (at >= 0 && at < n) ? s_id[at] : s_id[0];
    break;
  }
  Zout = Z;
  return tok;
}

// ----------------------------------------------------------------- draw unit
// Draw block (b, ch), ch < dchunks, of the decision-and-draw kernel: decision
// of sequence b, then the tile sums of slice ch of row pair n. Every block of
// a sampling sequence counts itself on the sequence's counter; the last one
// draws the token and returns the sequence's workspace entries to zero. A
// greedy sequence is decided by block 0 alone, and so is a filtered sequence
// whose target rows all have complete kept lists (block 0 then draws from
// the list and clears the sequence's entries; the other blocks leave at once).
template <int DT, bool VEC>
__device__ void draw_unit(const Params& P, int idx) {
  using Vc = Vec<DT, VEC>;
  constexpr int N = Vc::N;
  __shared__ Dec S;
  __shared__ int s_last;
  const int tid = threadIdx.x;
  // block order: every sequence's first block, then every sequence's second,
  // and so on, so that the first blocks (which draw alone when the kept lists
  // are complete) start together; no block of this kernel waits for another
  const int ch = idx / P.B;
  const int b = idx - ch * P.B;
  int d0, kb;
  if (!seq_bounds(P, b, d0, kb)) {
    if (ch == 0 && tid == 0) P.num_accepted[b] = SV_SEQ_BAD_OFFSETS;
    return;
  }
  const bool greedy = seq_greedy(P, b);
  if (greedy && ch != 0) return;  // one block decides a greedy sequence
  const bool lists = P.filt && P.kept != nullptr;
  // filtered: whether every target row's kept list is complete, so that the
  // draw, whichever row it takes, needs no tile sums. The first block resolves
  // it after its decision, so that the two sets of loads overlap; the others
  // leave at once when it holds.
  bool solo = false;
  int inc = 0;
  if (lists && !greedy) {
    for (int r = tid; r <= kb; r += kThreads)
      inc |= (int)P.kept[(size_t)(d0 + b + r) * kKeptWords + 1];
    if (ch != 0) {
      solo = __syncthreads_or(inc) == 0;
      if (solo) return;
    }
  }
  const Job j = decide<DT>(P, b, d0, kb, greedy, ch == 0, S);
  if (lists && !greedy && ch == 0) solo = __syncthreads_or(inc) == 0;
  if (greedy) {
    // the only reader of these partials returns them to zero
    __syncthreads();
    clear_partials(P, d0, kb, b, false);
    return;
  }
  // filtered: the kept lists of the sequence's target rows go back to zero
  // once this block has counted itself, spread over the blocks of the
  // sequence, except the list of the row drawn from (the last block clears it)
  const int keep_row = j.mode != kJobNone ? j.prow : -1;
  auto zero_list = [&](int row) {
    unsigned* kl = P.kept + (size_t)row * kKeptWords;
    const int words = 2 + 2 * (int)kl[0];
    __syncthreads();  // every thread has read the count
    for (int w = tid; w < words; w += kThreads) kl[w] = 0u;
  };
  auto zero_share = [&]() {
    if (!lists) return;
    for (int r = solo ? 0 : ch; r <= kb; r += solo ? 1 : P.dchunks)
      if (d0 + b + r != keep_row) zero_list(d0 + b + r);
  };
  // filtered: draw from the kept list when it holds the whole kept set
  const bool expl = lists && j.mode != kJobNone && explicit_usable(P, j);
  if (expl) {
    if (ch == 0) {
      float Z;
      const int tok = explicit_draw<DT>(P, j, Z);
      if (tid == 0) {
        pub_i(P.out_tokens + j.out_idx, tok);
        pub_i(P.num_accepted + b, j.n);
        if (P.diag.resid_Z) pub_f(P.diag.resid_Z + b, Z);
      }
    }
  } else if (j.mode != kJobNone) {
    // tile sums of slice ch of row pair n: the thread's vector k*kThreads + tid
    // of the slice belongs to tile ch*kTilesPerDraw + k
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
        float sum = 0.f;
#pragma unroll
        for (int k = 0; k < N; ++k) sum += draw_weight(fp[k], fq[k], j, P.c);
        ts[u] = sum;
      }
    }
    float tot[8];
    block_sum8(ts, tot);
    if (tid < kTilesPerDraw) {
      float val = tot[0];
#pragma unroll
      for (int k = 1; k < kTilesPerDraw; ++k) val = (tid == k) ? tot[k] : val;
      pub_f(P.tiles + (size_t)b * P.ntiles + ch * kTilesPerDraw + tid, val);
    }
  }
  // every block of the sequence counts itself, after its stores have landed
  if (!solo) {
    drain_stores();
    __syncthreads();
    if (tid == 0) s_last = (bump(P.draw_done + b) == P.dchunks - 1) ? 1 : 0;
    __syncthreads();
    if (!s_last) {
      zero_share();
      return;
    }
  }
  // Last block of the sequence: every other block has read the partials and
  // published its tile sums.
  if (j.mode != kJobNone && !expl) {
    float Z;
    const int tok = pick<DT, VEC>(P, b, j, Z);
    if (tid == 0) {
      pub_i(P.out_tokens + j.out_idx, tok);
      pub_i(P.num_accepted + b, j.n);
      if (P.diag.resid_Z) pub_f(P.diag.resid_Z + b, Z);
    }
  }
  __syncthreads();
  // return the sequence's workspace entries to zero
  if (!P.filt) clear_partials(P, d0, kb, b, true);
  if (P.filt) {
    zero_share();
    if (lists && keep_row >= 0) zero_list(keep_row);
    // the per-row filter results every block of the sequence has read
    for (int r = tid; r < 2 * kb + 1; r += kThreads) {
      const long long u = r < kb ? unit_of(P, false, d0 + r) : unit_of(P, true, d0 + b + (r - kb));
      P.rowres[u] = RowRes{0.f, 0.f, 0.f, 0};
    }
  }
  if (P.tok_logits != nullptr) {
    // LM-head path: the token logits of the sequence
    for (int r = tid; r < 2 * kb + 1; r += kThreads) {
      const long long u = r < kb ? unit_of(P, false, d0 + r) : unit_of(P, true, d0 + b + (r - kb));
      P.tok_logits[u] = 0.f;
    }
  }
  if (solo) return;  // no tile sums or counter were written
  for (int t = tid; t < P.ntiles; t += kThreads) pub_f(P.tiles + (size_t)b * P.ntiles + t, 0.f);
  if (tid == 0) pub_i(P.draw_done + b, 0);
}

// The decision-and-draw pass (filtered calls, and rows too long for k_verify).
template <int DT, bool VEC>
__global__ __launch_bounds__(kThreads) void k_draw(const Params P) {
  draw_unit<DT, VEC>(P, blockIdx.x);
}

__global__ void k_fill_zero(uint4* p, size_t n16) {
  for (size_t k = (size_t)blockIdx.x * blockDim.x + threadIdx.x; k < n16;
       k += (size_t)gridDim.x * blockDim.x)
    p[k] = make_uint4(0, 0, 0, 0);
}

// Records stage event i (if the caller passed that many).
static hipError_t stage_event(hipEvent_t* ev, int nev, int i, hipStream_t s) {
  return (ev != nullptr && i < nev) ? hipEventRecord(ev[i], s) : hipSuccess;
}

// Statistics, then (with top-k) the filter pass, then decision and draw. Stage
// events: before the first kernel, after each kernel of a filtered call (an
// unfiltered call here is one stage), and every further one after the last.
// Blocks of the filter launch: one row per wave.
static unsigned filter_grid(const Plan& L) {
  return (unsigned)((L.filter_blocks + kFiltRowsPerBlock - 1) / kFiltRowsPerBlock);
}

template <int DT, bool VEC>
static hipError_t launch_t(const Params& P, const Plan& L, hipStream_t s, hipEvent_t* ev, int nev) {
  hipError_t err;
  int e = 0;
  if ((err = stage_event(ev, nev, e++, s)) != hipSuccess) return err;
  if (P.filt) {
    if (P.nucleus)
      hipLaunchKernelGGL((k_stats<DT, VEC, false>), dim3((unsigned)L.stats_blocks), dim3(kThreads),
                         0, s, P);
    else
      hipLaunchKernelGGL((k_stats<DT, VEC, true>), dim3((unsigned)L.stats_blocks), dim3(kThreads),
                         0, s, P);
    if ((err = hipGetLastError()) != hipSuccess) return err;
    if ((err = stage_event(ev, nev, e++, s)) != hipSuccess) return err;
    if (P.nucleus)
      hipLaunchKernelGGL((k_nucleus<DT, VEC>), dim3((unsigned)L.filter_blocks), dim3(kNucThreads),
                         0, s, P);
    else
      hipLaunchKernelGGL(k_filter<DT>, dim3(filter_grid(L)), dim3(kThreads), 0, s, P);
    if ((err = hipGetLastError()) != hipSuccess) return err;
    if ((err = stage_event(ev, nev, e++, s)) != hipSuccess) return err;
  } else {
    hipLaunchKernelGGL((k_stats<DT, VEC, false>), dim3((unsigned)L.stats_blocks), dim3(kThreads),
                       0, s, P);
    if ((err = hipGetLastError()) != hipSuccess) return err;
  }
  hipLaunchKernelGGL((k_draw<DT, VEC>), dim3((unsigned)L.draw_blocks), dim3(kThreads), 0, s, P);
  if ((err = hipGetLastError()) != hipSuccess) return err;
  // this and any further events: after the last kernel
  for (; e < nev; ++e)
    if ((err = stage_event(ev, nev, e, s)) != hipSuccess) return err;
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

template <int DT, bool VEC>
static hipError_t launch_row_stats_t(const Params& P, const Plan& L, hipStream_t s) {
  if (P.nucleus) {
    hipLaunchKernelGGL((k_stats<DT, VEC, false>), dim3((unsigned)L.stats_blocks), dim3(kThreads),
                       0, s, P);
    hipError_t err = hipGetLastError();
    if (err != hipSuccess) return err;
    hipLaunchKernelGGL((k_nucleus<DT, VEC>), dim3((unsigned)L.filter_blocks), dim3(kNucThreads), 0,
                       s, P);
  } else if (P.filt) {
    hipLaunchKernelGGL((k_stats<DT, VEC, true>), dim3((unsigned)L.stats_blocks), dim3(kThreads), 0,
                       s, P);
    hipError_t err = hipGetLastError();
    if (err != hipSuccess) return err;
    hipLaunchKernelGGL(k_filter<DT>, dim3(filter_grid(L)), dim3(kThreads), 0, s, P);
  } else {
    hipLaunchKernelGGL((k_stats<DT, VEC, false>), dim3((unsigned)L.stats_blocks), dim3(kThreads),
                       0, s, P);
  }
  return hipGetLastError();
}

hipError_t launch_row_stats(int dtype, bool vec, const Params& P, const Plan& L, hipStream_t s) {
  switch (dtype) {
    case SV_F32:
      return vec ? launch_row_stats_t<SV_F32, true>(P, L, s) : launch_row_stats_t<SV_F32, false>(P, L, s);
    case SV_F16:
      return vec ? launch_row_stats_t<SV_F16, true>(P, L, s) : launch_row_stats_t<SV_F16, false>(P, L, s);
    default:
      return vec ? launch_row_stats_t<SV_BF16, true>(P, L, s) : launch_row_stats_t<SV_BF16, false>(P, L, s);
  }
}

hipError_t launch_draw_f32(bool vec, const Params& P, const Plan& L, hipStream_t s) {
  if (vec)
    hipLaunchKernelGGL((k_draw<SV_F32, true>), dim3((unsigned)L.draw_blocks), dim3(kThreads), 0, s,
                       P);
  else
    hipLaunchKernelGGL((k_draw<SV_F32, false>), dim3((unsigned)L.draw_blocks), dim3(kThreads), 0, s,
                       P);
  return hipGetLastError();
}

hipError_t fill_zero(void* p, size_t bytes, hipStream_t s) {
  const size_t n16 = bytes / 16;
  if (n16 == 0) return hipSuccess;
  const unsigned blocks = (unsigned)((n16 + 255) / 256 < 1024 ? (n16 + 255) / 256 : 1024);
  hipLaunchKernelGGL(k_fill_zero, dim3(blocks), dim3(256), 0, s, reinterpret_cast<uint4*>(p), n16);
  return hipGetLastError();
}

}  // namespace sv
