// The unfiltered verification step as one HIP kernel for gfx950.
//
// Grid: the statistics blocks and D draw blocks per sequence. A dense batch
// streams its rows position-major (every sequence's position 0, then position
// 1, ...), so a sequence that stops early is decided while the rows of later
// positions still stream. When the chip can hold every draw block at once with
// room to spare, the draw blocks sit before the statistics of the last two
// positions, whose rows only sequences that accept nearly every draft need:
// the draws then overlap the end of the stream. Otherwise they follow all the
// statistics.
//
// A statistics block streams one chunk of one logit row and publishes one
// 64-bit partial: for a sampling row the chunk maximum m and the sum of
// 2^(l*c - R), R = fp32(m*c); for a greedy row the chunk argmax and whether the
// chunk holds NaN or +inf. Statistics blocks never wait.
//
// Draw block (b, s) takes slice s (kDrawVecs vectors) of the vocabulary of
// sequence b. Thread j merges the partials of position j in chunk order as they
// are published and decides the position: r_j = p_j(x_j)/q_j(x_j), accept iff
// u_j < r_j. The first stop n (a rejection, an invalid row or id, or the bonus
// position) ends the walk; every draw block of the sequence reaches the same n
// with the same arithmetic, so no decision is broadcast, and block 0 writes the
// accepted prefix. For the final draw each block loads its slice of row pair n
// into registers, forms the weights max(0, p_n - q_n) (or p_n for the bonus),
// and publishes the slice's weight sum; each block gathers all slice sums, and
// the block whose slice holds u*Z scans its own registers for the token, in
// ascending id order.
//
// Deadlock freedom: blocks start in index order on each of the chip's dies and
// statistics blocks never wait. Draw blocks placed ahead of statistics they may
// wait for number fewer than the chip holds at once, less one block per compute
// unit, so those statistics always find room; a draw block waits for the other
// draw blocks of its sequence only after its own slice is published, and they
// are consecutive in the grid. Every wait is bounded anyway
// (SV_SEQ_SYNC_TIMEOUT).
//
// Pages (by title, section): aivaro.ru answer 289 "Как работает speculative
// decoding на уровне логитов, а не токенов?" s.5 steps 3-4, s.6, s.9 (softmax
// of both rows, ratio test with "<", truncation at the first rejection,
// residual max(0, p - q)/Z, multinomial draw); Hung-yi Lee lecture-16 notes
// part "4、推测解码验证流程图" items 1-4 (one target pass scores every
// position, position-by-position check, truncation, bonus token); aihero.vn
// "Speculative decoding" sections "Chấp nhận bằng tỉ lệ, không chỉ bằng argmax"
// (q draft, p target at the same prefix, ratio, residual) and "Cùng phân bố
// không có nghĩa cùng chuỗi mỗi lần" (greedy check, consistent temperature).
#include "sv_rows.h"

namespace sv {

namespace {

constexpr int kPollGroup = 4;   // chunk partials a deciding thread reads per round
constexpr int kPollSleep = 8;   // s_sleep units (64 clocks each) between rounds

// Block-shared state of a draw block.
struct DrawShared {
  float mq[SV_MAX_K + 1], sq[SV_MAX_K + 1];  // merged draft-row statistics by position
  float mp[SV_MAX_K + 1], sp[SV_MAX_K + 1];  // merged target-row statistics
  int am[SV_MAX_K + 1];                      // greedy: merged target argmax
  int first;    // first stopping position (rejection, invalid row or id, the
                // bonus position)
  int invalid;  // first position with an invalid row
  int to_pos;   // first position whose wait ran out
  int badtok;   // a draft id outside [0, V) anywhere in the sequence
  int last;     // this block is the sequence's last to finish
  int flags;    // the sequence's kSeqFlag bits, read by the last block
};

// Draw weight of one id for rows without a filter: max(0, p - q) for the
// residual, p for the bonus (every id is in both kept sets).
__device__ __forceinline__ float weight(float lp, float lq, const Job& j, float c) {
  const float ep = fast_exp2(fmaf(lp, c, -j.Rp));
  if (j.mode == kJobBonus) return ep * j.invSp;
  return fmaxf(fmaf(ep, j.invSp, -fast_exp2(fmaf(lq, c, -j.Rq)) * j.invSq), 0.0f);
}

__device__ __forceinline__ unsigned long long tag_sum(float z) {
  return (1ull << 63) | (unsigned long long)__float_as_uint(z);
}

// Tile sums of the draw weights of this block's slice (every thread gets all
// kTilesPerDraw tile totals) and their sum in tile order.
template <int DT, bool VEC, class Raw>
__device__ __forceinline__ float slice_weights(const Raw (&rp)[kTilesPerDraw],
                                               const Raw (&rq)[kTilesPerDraw], int vb, int nvec,
                                               const Job& j, float c,
                                               float (&tot)[kTilesPerDraw]) {
  using Vc = Vec<DT, VEC>;
  constexpr int N = Vc::N;
  float ts[kTilesPerDraw];
#pragma unroll
  for (int k = 0; k < kTilesPerDraw; ++k) {
    ts[k] = 0.f;
    if (vb + k * kThreads < nvec) {
      float fp[N], fq[N];
      Vc::get(rp[k], fp);
      if (j.mode == kJobResidual) {
        Vc::get(rq[k], fq);
      } else {
#pragma unroll
        for (int e = 0; e < N; ++e) fq[e] = 0.f;
      }
      float sum = 0.f;
#pragma unroll
      for (int e = 0; e < N; ++e) sum += weight(fp[e], fq[e], j, c);
      ts[k] = sum;
    }
  }
  block_sum<kTilesPerDraw>(ts, tot);
  float z = 0.f;
#pragma unroll
  for (int k = 0; k < kTilesPerDraw; ++k) z += tot[k];
  return z;
}

// Waits (bounded) for the D published slice sums at `p`: thread k < D returns
// sum k (0 elsewhere). Sets `to` in every thread if a wait ran out.
__device__ float gather_sum(const Params& P, const unsigned long long* p, int D, int& to) {
  float z = 0.f;
  int t = 0;
  if ((int)threadIdx.x < D) {
    unsigned long long v = obs_u64(p + threadIdx.x);
    for (int spins = 0; v == 0ull; ++spins) {
      if (spins >= P.spin_limit) {
        t = 1;
        break;
      }
      __builtin_amdgcn_s_sleep(2);
      v = obs_u64(p + threadIdx.x);
    }
    z = __uint_as_float((unsigned)v);
  }
  to = __syncthreads_or(t);
  return z;
}

// The final draw of sequence b (every draw block of the sequence; whole block).
// Returns the token in the block whose slice holds the crossing, -1 elsewhere;
// Z receives the mass normalised by. Sets `to` on a timed-out wait.
template <int DT, bool VEC>
__device__ int slice_draw(const Params& P, Job j, int b, int s, float& Z, int& to) {
  using Vc = Vec<DT, VEC>;
  constexpr int N = Vc::N;
  __shared__ float s_base;
  __shared__ int s_slice, s_tok;
  const int tid = threadIdx.x;
  const int D = P.dchunks;
  const int vb = s * kDrawVecs + tid;
  const size_t prow = (size_t)j.prow * P.V;
  const size_t qrow = (size_t)j.qrow * P.V;
  typename Vc::Raw rp[kTilesPerDraw], rq[kTilesPerDraw];
#pragma unroll
  for (int k = 0; k < kTilesPerDraw; ++k) {
    const int v = vb + k * kThreads;
    rp[k] = rq[k] = typename Vc::Raw{};
    if (v < P.nvec) {
      rp[k] = Vc::load(P.target, prow, v);
      if (j.mode == kJobResidual) rq[k] = Vc::load(P.draft, qrow, v);
    }
  }
  unsigned long long* sums = P.draws + (size_t)b * 2 * D;
  float tot[kTilesPerDraw];
  float zs = slice_weights<DT, VEC>(rp, rq, vb, P.nvec, j, P.c, tot);
  if (tid == 0) pub_u64(sums + s, tag_sum(zs));
  float zk = gather_sum(P, sums, D, to);
  if (to) return -1;
  float incl = block_incl_scan(zk, Z);  // thread k: slices 0..k (k < D)
  if (!(Z > 0.f) && j.mode == kJobResidual) {
    // The residual mass rounded to zero (a rejection implies Z > 0 in exact
    // arithmetic): draw from p_n instead.
    j.mode = kJobBonus;
    zs = slice_weights<DT, VEC>(rp, rq, vb, P.nvec, j, P.c, tot);
    if (tid == 0) pub_u64(sums + D + s, tag_sum(zs));
    zk = gather_sum(P, sums + D, D, to);
    if (to) return -1;
    incl = block_incl_scan(zk, Z);
  }
  const float target = j.u * Z;
  // the slice holding the crossing: the first whose inclusive prefix exceeds
  // u*Z, else (rounding) the last slice with mass
  int cs = block_first_lane(tid < D && incl > target);
  if (cs == INT_MAX) cs = block_last_lane(tid < D && zk > 0.f);
  if (cs < 0) cs = 0;
  if (tid == cs) {
    s_slice = cs;
    s_base = incl - zk;
  }
  __syncthreads();
  if (s_slice != s) return -1;
  const float base = s_base;
  // the tile of this slice holding the crossing (same rule)
  int ks = -1, klast = -1;
  float tbase = 0.f, tlast = 0.f, run = base;
#pragma unroll
  for (int k = 0; k < kTilesPerDraw; ++k) {
    const float nx = run + tot[k];
    if (ks < 0 && nx > target) {
      ks = k;
      tbase = run;
    }
    if (tot[k] > 0.f) {
      klast = k;
      tlast = run;
    }
    run = nx;
  }
  if (ks < 0) {
    ks = klast < 0 ? 0 : klast;
    tbase = klast < 0 ? base : tlast;
  }
  // scan of tile ks: thread t owns vector vb + ks*kThreads (ascending ids)
  const int v = vb + ks * kThreads;
  float fp[N], fq[N];
#pragma unroll
  for (int e = 0; e < N; ++e) fp[e] = fq[e] = 0.f;
#pragma unroll
  for (int k = 0; k < kTilesPerDraw; ++k) {
    if (k == ks) {
      Vc::get(rp[k], fp);
      if (j.mode == kJobResidual) Vc::get(rq[k], fq);
    }
  }
  if (j.mode != kJobResidual) {
#pragma unroll
    for (int e = 0; e < N; ++e) fq[e] = 0.f;
  }
  float w[N];
  float acc = 0.f;
#pragma unroll
  for (int e = 0; e < N; ++e) {
    acc += (v < P.nvec) ? weight(fp[e], fq[e], j, P.c) : 0.f;
    w[e] = acc;
  }
  float total;
  const float excl = tbase + (block_incl_scan(acc, total) - acc);
  // the first thread whose cumulative weight passes u*Z holds the token; if
  // rounding leaves none, the last positive weight of the tile
  const int tc = block_first_lane(excl + acc > target);
  if (tc != INT_MAX) {
    if (tid == tc) {
      int e = 0;
      while (e < N - 1 && !(excl + w[e] > target)) ++e;
      s_tok = v * N + e;
    }
  } else {
    const int tl = block_last_lane(acc > 0.f);
    if (tid == (tl < 0 ? 0 : tl)) {
      int e = N - 1;
      while (e > 0 && !(w[e] > w[e - 1])) --e;
      s_tok = tl < 0 ? (s * kDrawVecs + ks * kThreads) * N : v * N + e;
    }
  }
  __syncthreads();
  return s_tok;
}

// Returns the partials of a sequence's rows to zero (whole block): its target
// rows and, with_draft, its draft rows. A row the decision never read may still
// be in flight: its partial is awaited first. Returns nonzero (in every
// thread) if such a wait ran out. With keep_pairs only the bonus row's
// partials are cleared: the acceptance statistics pass reads the others next
// (it clears them, and the kernel boundary orders it after every publish).
__device__ int clear_partials(const Params& P, int d0, int kb, int b, bool with_draft,
                              bool keep_pairs = false) {
  const int C = P.chunks;
  const int nd = with_draft ? kb : 0;
  const int first = keep_pairs ? nd + kb : 0;  // the bonus row is row nd + kb
  int to = 0;
  for (int k = threadIdx.x + first * C; k < (nd + kb + 1) * C; k += kThreads) {
    const int r = k / C, ch = k - r * C;
    const bool tgt = r >= nd;
    unsigned long long* p =
        P.slots + unit_of(P, tgt, tgt ? d0 + b + (r - nd) : d0 + r) * C + ch;
    for (int spins = 0; obs_u64(p) == 0ull; ++spins) {
      if (spins >= P.spin_limit) {
        to = 1;
        break;
      }
      __builtin_amdgcn_s_sleep(4);
    }
    pub_u64(p, 0ull);
  }
  return __syncthreads_or(to);
}

// Counts this block on sequence b's counter once its stores have landed
// (whole block; `total` blocks take part). The last one returns the sequence's
// partials (awaiting rows still in flight), slice sums, counter and flags to
// zero, and reports a timed-out wait.
__device__ void finish_sequence(const Params& P, int b, int d0, int kb, bool greedy, int total,
                                int seq_to, DrawShared& S) {
  const int tid = threadIdx.x;
  const int D = P.dchunks;
  const int t0 = d0 + b;
  if (tid == 0 && seq_to) raise_flag(P.seq_flags + b, kSeqFlagTimeout);
  drain_stores();
  __syncthreads();
  if (tid == 0) {
    S.last = (bump(P.draw_done + b) == total - 1) ? 1 : 0;
    compiler_fence();
    S.flags = S.last ? obs_i(P.seq_flags + b) : 0;
  }
  __syncthreads();
  if (!S.last) return;
  const int cto = clear_partials(P, d0, kb, b, !greedy, P.keep_pair_partials && !greedy);
  if ((S.flags & kSeqFlagTimeout) || cto) {
    for (int k = tid; k <= kb; k += kThreads) pub_i(P.out_tokens + t0 + k, -1);
    if (tid == 0) {
      pub_i(P.num_accepted + b, SV_SEQ_SYNC_TIMEOUT);
      if (P.diag.resid_Z) pub_f(P.diag.resid_Z + b, __builtin_nanf(""));
    }
  }
  for (int k = tid; k < 2 * D; k += kThreads) pub_u64(P.draws + (size_t)b * 2 * D + k, 0ull);
  if (tid == 0) {
    pub_i(P.seq_flags + b, 0);
    pub_i(P.draw_done + b, 0);
  }
}

// Draw block s of sequence b (see the file comment). A greedy sequence is
// decided by its block 0 alone.
template <int DT, bool VEC>
__device__ void draw_block(const Params& P, int idx) {
  __shared__ DrawShared S;
  const int tid = threadIdx.x;
  const int C = P.chunks;
  const int D = P.dchunks;
  const float c = P.c;
  const int b = idx / D;
  const int s = idx - b * D;
  int d0, kb;
  if (!seq_bounds(P, b, d0, kb)) {
    if (s == 0 && tid == 0) P.num_accepted[b] = SV_SEQ_BAD_OFFSETS;
    return;
  }
  const bool greedy = seq_greedy(P, b);
  if (greedy && s != 0) return;
  const int t0 = d0 + b;

  // decision inputs (the logits at the draft ids are loaded before any wait)
  int x = -1;
  float u = 1.f;
  if (tid < kb) {
    x = P.tokens[d0 + tid];
    if (!greedy) u = P.uniforms[t0 + tid];
  }
  const float u_draw = greedy ? 0.f : P.uniforms[t0 + kb];
  const bool tok_ok = tid >= kb || (x >= 0 && x < P.V);
  float lq = 0.f, lp = 0.f;
  if (tid < kb && !greedy) {
    const int xs = tok_ok ? x : 0;
    lq = load_elem<DT>(P.draft, (size_t)(d0 + tid) * P.V + xs);
    lp = load_elem<DT>(P.target, (size_t)(t0 + tid) * P.V + xs);
  }
  if (tid == 0) {
    S.first = INT_MAX;
    S.invalid = INT_MAX;
    S.to_pos = INT_MAX;
    S.badtok = 0;
  }
  __syncthreads();
  if (tid < kb && !tok_ok) atomicOr(&S.badtok, 1);  // every draft id is checked

  // Thread j merges position j's partials in chunk order as they are published
  // and decides the position as soon as it has them all, inside the polling
  // loop, so the other threads of its wave see a stop on their next round. A
  // position past an already-known stop needs no statistics (unless side
  // outputs want every row).
  float mq = kNegInf, sq = 0.f, mp = kNegInf, sp = 0.f;
  float ratio = __builtin_nanf("");
  int am = INT_MAX;
  int to = 0;
  if (tid <= kb) {
    const bool wq = !greedy && tid < kb;
    const unsigned long long* tsl = P.slots + unit_of(P, true, t0 + tid) * C;
    const unsigned long long* dsl = wq ? P.slots + unit_of(P, false, d0 + tid) * C : tsl;
    const volatile int* vfirst = &S.first;
    int k0 = 0, gbad = 0;
    for (int spins = 0;; ++spins) {
      unsigned long long tv[kPollGroup], dv[kPollGroup];
#pragma unroll
      for (int gg = 0; gg < kPollGroup; ++gg) {
        const bool in = k0 + gg < C;
        tv[gg] = in ? obs_u64(tsl + k0 + gg) : 0ull;
        dv[gg] = (in && wq) ? obs_u64(dsl + k0 + gg) : 1ull;
      }
      int adv = 0;
      bool ok = true;
#pragma unroll
      for (int gg = 0; gg < kPollGroup; ++gg) {
        if (ok && k0 + gg < C) {
          if (tv[gg] == 0ull || dv[gg] == 0ull) {
            ok = false;
          } else {
            float m, s_;
            if (greedy) {
              int ci, cb;
              unpack_am(tv[gg], m, ci, cb);
              argmax_merge(mp, am, m, ci);
              gbad |= cb;
            } else {
              if (wq) {
                unpack_ms(dv[gg], m, s_);
                merge_ms(mq, sq, m, s_, c);
              }
              unpack_ms(tv[gg], m, s_);
              merge_ms(mp, sp, m, s_, c);
            }
            ++adv;
          }
        }
      }
      k0 += adv;
      if (k0 >= C) {
        // position tid: valid rows, then the accept test (the bonus position
        // and an invalid id always stop the walk)
        bool valid, acc = false;
        if (greedy) {
          valid = !gbad && mp != kNegInf;
        } else {
          valid = __builtin_isfinite(mp) && sp > 0.f && __builtin_isfinite(sp);
          if (wq) valid = valid && __builtin_isfinite(mq) && sq > 0.f && __builtin_isfinite(sq);
        }
        if (tid < kb && tok_ok && valid) {
          if (greedy) {
            acc = am == x;
          } else {
            // r = p(x)/q(x) = 2^((lp*c - Rp) - (lq*c - Rq)) * Sq / Sp; q(x) = 0 < p(x)
            // gives +inf (accept), q(x) = p(x) = 0 gives NaN (reject)
            const float ep = fmaf(lp, c, -ref_of(mp, c));
            const float eq = fmaf(lq, c, -ref_of(mq, c));
            ratio = fast_exp2(ep - eq) * (sq / sp);
            acc = u < ratio;  // strict: u == r rejects
          }
        }
        S.mq[tid] = mq;
        S.sq[tid] = sq;
        S.mp[tid] = mp;
        S.sp[tid] = sp;
        S.am[tid] = am;
        if (!valid) atomicMin(&S.invalid, tid);
        if (!acc) atomicMin(&S.first, tid);
        break;
      }
      if (!P.full_wait && *vfirst < tid) break;
      if (spins >= P.spin_limit) {
        to = 1;
        break;
      }
      __builtin_amdgcn_s_sleep(kPollSleep);
    }
  }
  if (to) atomicMin(&S.to_pos, tid);
  __syncthreads();
  const int first = S.first;
  const int n = min(first, kb);
  // a wait that ran out matters if its position is reached (or no stop was seen)
  const int code = (S.to_pos != INT_MAX && S.to_pos <= first) ? SV_SEQ_SYNC_TIMEOUT
                   : S.badtok                                 ? SV_SEQ_BAD_TOKEN
                   : (S.invalid == n)                         ? SV_SEQ_BAD_ROW
                                                              : 0;
  const bool draws = code == 0 && !greedy;

  int seq_to = code == SV_SEQ_SYNC_TIMEOUT ? 1 : 0;

  if (s == 0) {
    // The writer block: the accepted prefix, -1 after n, slot n when nothing
    // is drawn, and the side outputs. Outputs a later timeout report may
    // overwrite are written with agent-scope stores, so they land before this
    // block counts itself.
    if (tid <= kb && !(draws && tid == n)) {
      int tok = -1;
      if (code == 0) {
        if (tid < n) tok = x;
        else if (tid == n) tok = S.am[n];
      }
      pub_i(P.out_tokens + t0 + tid, tok);
    }
    if (tid == 0 && !draws) {
      pub_i(P.num_accepted + b, code ? code : n);
      if (P.diag.resid_Z) pub_f(P.diag.resid_Z + b, __builtin_nanf(""));
    }
    if (tid <= kb) {
      const float kLn2 = 0.69314718055994531f;
      const float nan = __builtin_nanf("");
      if (P.diag.row_max_target) P.diag.row_max_target[t0 + tid] = mp;
      if (P.diag.row_logsum_target)
        P.diag.row_logsum_target[t0 + tid] =
            greedy ? nan : (__log2f(sp) + fmaf(-mp, c, ref_of(mp, c))) * kLn2;
      if (tid < kb) {
        if (P.diag.row_max_draft) P.diag.row_max_draft[d0 + tid] = greedy ? nan : mq;
        if (P.diag.row_logsum_draft)
          P.diag.row_logsum_draft[d0 + tid] =
              greedy ? nan : (__log2f(sq) + fmaf(-mq, c, ref_of(mq, c))) * kLn2;
        if (P.diag.ratio) P.diag.ratio[d0 + tid] = ratio;
      }
    }
  }
  if (draws) {
    Job j;
    j.mode = n < kb ? kJobResidual : kJobBonus;
    j.n = n;
    j.prow = t0 + n;
    j.qrow = d0 + n;
    j.Rq = ref_of(S.mq[n], c);
    j.invSq = 1.0f / S.sq[n];
    j.Rp = ref_of(S.mp[n], c);
    j.invSp = 1.0f / S.sp[n];
    j.thr_q = kNegInf;
    j.thr_p = kNegInf;
    j.u = u_draw;
    j.out_idx = t0 + n;
    float Z = 0.f;
    int dto = 0;
    const int tok = slice_draw<DT, VEC>(P, j, b, s, Z, dto);
    seq_to |= dto;
    if (tok >= 0 && tid == 0) {
      pub_i(P.out_tokens + t0 + n, tok);
      pub_i(P.num_accepted + b, n);
      if (P.diag.resid_Z) pub_f(P.diag.resid_Z + b, Z);
    }
  }
  finish_sequence(P, b, d0, kb, greedy, greedy ? 1 : D, seq_to, S);
}

// Row and chunk of statistics block g. Dense batches stream position-major:
// every sequence's position-0 rows (draft then target, chunks innermost), then
// position 1, ..., then the bonus rows, so a sequence that stops early has its
// statistics early. Ragged batches stream the draft rows, then the target
// rows. Greedy-only calls skip the draft rows.
__device__ __forceinline__ void stats_row(const Params& P, long long g, bool& is_target, int& row,
                                          int& ch) {
  const long long C = P.chunks;
  if (P.cu == nullptr) {
    const int B = P.B, K = P.K;
    const long long per = (P.all_greedy ? 1LL : 2LL) * B * C;  // blocks per position < K
    const int j = (int)min((long long)K, g / per);
    long long r = g - (long long)j * per;
    if (j < K && !P.all_greedy) {
      const int b = (int)(r / (2 * C));
      r -= (long long)b * 2 * C;
      is_target = r >= C;
      ch = (int)(is_target ? r - C : r);
      row = is_target ? b * (K + 1) + j : b * K + j;
    } else {
      const int b = (int)(r / C);
      ch = (int)(r - (long long)b * C);
      is_target = true;
      row = b * (K + 1) + j;
    }
    return;
  }
  const long long unit = (g + P.stats_block0) / C;
  ch = (int)(g + P.stats_block0 - unit * C);
  row_of_unit(P, (int)unit, is_target, row);
}

// Statistics block g (see stats_row), published with an agent-scope store for
// the draw blocks of the same grid.
template <int DT, bool VEC>
__device__ void stats_block(const Params& P, long long g) {
  __shared__ int s_cu[kCuLds];
  bool is_target;
  int row, ch;
  stats_row(P, g, is_target, row, ch);
  bool greedy = P.all_greedy != 0;
  if (!greedy && P.greedy != nullptr) greedy = P.greedy[row_seq(P, row, is_target, s_cu)] != 0;
  if (greedy && !is_target) return;  // greedy sequences never read draft rows
  const void* base = is_target ? P.target : P.draft;
  const int vb = ch * P.chunk_vecs;
  // Position 0's rows are the ones draws re-read most often (most rejections
  // come first): ordinary loads leave them in the last-level cache; the rest
  // stream.
  const bool first = P.cu == nullptr && (is_target ? row % (P.K + 1) : row % max(P.K, 1)) == 0;
  const unsigned long long packed = chunk_stats<DT, VEC>(
      P, base, (size_t)row * (size_t)P.V, vb, min(P.nvec, vb + P.chunk_vecs), greedy, !first);
  if (threadIdx.x == 0) pub_u64(P.slots + unit_of(P, is_target, row) * P.chunks + ch, packed);
}

// Waves per SIMD asked of the compiler: bf16 and fp32 rows fit 64 VGPRs
// without spills (eight blocks per compute unit); fp16 rows, whose unpacking
// costs more registers, are left to the compiler.
template <int DT>
constexpr int kVerifyWaves = DT == SV_BF16 ? 8 : (DT == SV_F32 ? 7 : 1);

template <int DT, bool VEC>
__global__ __launch_bounds__(kThreads, kVerifyWaves<DT>) void k_verify(const Params P) {
  // Grid order: statistics blocks up to draw_at, the draw blocks, the remaining
  // statistics blocks (one call site per block kind, so both inline).
  long long g = blockIdx.x;
  const long long nd = (long long)P.B * P.dchunks;
  bool stats = true;
  if (g >= P.draw_at) {
    if (g < P.draw_at + nd) {
      stats = false;
      g -= P.draw_at;
    } else {
      g -= nd;
    }
  }
  if (stats) stats_block<DT, VEC>(P, g);
  else draw_block<DT, VEC>(P, (int)g);
}

template <int DT, bool VEC>
hipError_t launch_t(const Params& P, const Plan& L, hipStream_t s) {
  hipLaunchKernelGGL((k_verify<DT, VEC>), dim3((unsigned)(L.stats_blocks + L.draw_blocks)),
                     dim3(kThreads), 0, s, P);
  return hipGetLastError();
}

template <int DT, bool VEC>
long long capacity_t(int cus) {
  int per_cu = 0;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, k_verify<DT, VEC>, kThreads, 0) !=
      hipSuccess)
    return 0;
  return (long long)per_cu * cus;
}

}  // namespace

long long fused_capacity(int dtype, bool vec, int cus) {
  switch (dtype) {
    case SV_F32: return vec ? capacity_t<SV_F32, true>(cus) : capacity_t<SV_F32, false>(cus);
    case SV_F16: return vec ? capacity_t<SV_F16, true>(cus) : capacity_t<SV_F16, false>(cus);
    default: return vec ? capacity_t<SV_BF16, true>(cus) : capacity_t<SV_BF16, false>(cus);
  }
}

hipError_t launch_fused(int dtype, bool vec, const Params& P, const Plan& L, hipStream_t s) {
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
