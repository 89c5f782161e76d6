// Verification of several draft chains per sequence for gfx950
// (spec_verify_multi).
//
// M chains of K drafts share one prefix; chain m's rows at position j are
// conditioned on that chain's own tokens. The row statistics of every draft
// and target row come from the statistics pass of the single-chain path
// (k_stats, the chains laid out as B*M sequences). Then k_multi runs
// kMultiSplit blocks of 1024 threads per sequence, each on a contiguous range
// of the vocabulary's tiles; every block walks the sequence the same way and
// the blocks exchange their pass sums through the workspace. It walks the
// positions: the chains still alive are those whose tokens so far equal the
// emitted ones. Their candidates at position j are
// tested in chain order against the current law r, starting from the lowest
// live chain's target row p_j: accept iff u < r(x)/q_m(x). After a rejection
// the law becomes max(0, r - q_m)/Z, one pass over the vocabulary for Z. The
// next candidate is tested against it. An accepted token keeps the chains
// that proposed it and moves to the next position. When every candidate is
// rejected (or at the bonus position), the token is drawn from the current
// law by inverse CDF in ascending id order: one pass for per-tile sums, then
// a scan of the crossing tile. The law of an id is p(x) with each rejected
// candidate's q peeled off in turn, so no law is ever stored.
//
// Pages (by title, section): aivaro.ru answer 289 "Как работает speculative
// decoding на уровне логитов, а не токенов?" s.6 (accept min(1, p/q), else
// draw from max(0, p - q)/Z: rejection sampling whose result follows p),
// s.5 steps 3-4 (truncation); Hung-yi Lee lecture-16 notes part "1、第16講"
// (there can be several drafters) and part "4、推测解码验证流程图" item 4
// (bonus token); aihero.vn "Speculative decoding" section "Chấp nhận bằng tỉ
// lệ, không chỉ bằng argmax" (q draft, p target at the same prefix).
#include "sv_rows.h"

namespace sv {

namespace {

// A block of 1024 threads walks one sequence: each pass over the vocabulary
// streams its rows with every thread of a whole compute unit, which the walk
// (one block per sequence, B blocks) needs to keep enough loads in flight.
constexpr int kMT = 1024;               // threads of a k_multi block
constexpr int kMW = kMT / kWave;        // its waves
constexpr int kMTile = kMT;             // vectors of a draw tile: one per thread
constexpr int kMultiMaxTiles = kMultiMaxVecs / kMTile;  // tiles a row may have

// Tiles a thread has in flight per round of a pass that loads R rows at each
// vector: about eight vector loads per thread whatever the number of rows.
__host__ __device__ constexpr int multi_batch(int R) { return R <= 1 ? 8 : (R == 2 ? 4 : 2); }

struct RowS {
  float R, iS;  // reference R = fp32(max*c) and 1/S of the row's (kept) sum of 2^(l*c - R)
  float thr;    // kept set: l >= thr (-inf without filters)
  int ok;       // the row holds no NaN or +inf and some finite value
};

// Probability of logit l in a row: 2^(l*c - R) / S inside its kept set, 0
// outside (FILT: the row has a cut; without one every id is kept).
template <bool FILT>
__device__ __forceinline__ float prob_of(float l, const RowS& r, float c) {
  const float v = fast_exp2(fmaf(l, c, -r.R)) * r.iS;
  if constexpr (FILT) return l >= r.thr ? v : 0.f;
  return v;
}

// Statistics of one row: with filters the kept-set maximum, sum and threshold
// of the cut pass; otherwise its chunk partials merged in chunk order.
__device__ __forceinline__ RowS merged_row(const Params& P, long long unit) {
  RowS r;
  if (P.filt) {
    const RowRes rr = P.rowres[unit];
    r.ok = rr.flags == 0 && __builtin_isfinite(rr.m) && rr.s > 0.f && __builtin_isfinite(rr.s);
    r.R = ref_of(rr.m, P.c);
    r.iS = 1.0f / rr.s;
    r.thr = rr.theta;
    return r;
  }
  float m = kNegInf, s = 0.f;
  const unsigned long long* sl = P.slots + unit * P.chunks;
  for (int k = 0; k < P.chunks; ++k) {
    float om, os;
    unpack_ms(sl[k], om, os);
    merge_ms(m, s, om, os, P.c);
  }
  r.ok = __builtin_isfinite(m) && s > 0.f && __builtin_isfinite(s);
  r.R = ref_of(m, P.c);
  r.iS = 1.0f / s;
  r.thr = kNegInf;
  return r;
}

struct MultiShared {
  float tsum[kMultiMaxTiles][kMW];  // per-tile, per-wave sums of a draw pass
  float red[kMW];              // block reductions
  int redi[kMW];
  RowS p;                      // the node's target row
  RowS q[SV_MAX_CHAINS];       // the rejected candidates' draft rows, in order
  int qrow[SV_MAX_CHAINS];     // their draft rows
  float iZ[SV_MAX_CHAINS];     // 1/Z of each remainder
  int nrej;
  int prow;                    // the node's target row
  int pok;                     // the node's target row is usable
  // thread 0's decisions, read by the whole block
  int act;                     // 1 accepted, 2 rejected, 4 an unusable draft row
  int xrow;                    // draft row of the candidate under test
  RowS xq;                     // its statistics
  float base;                  // mass before the crossing tile
  float target;                // u * Z of the draw
  int ct;                      // the crossing tile
  int tok;                     // the drawn token
  int tb, te;                  // this block's tiles of every pass
  int pass;                    // passes this block has joined
  int to;                      // a wait of this block ran out
};

// Cross-block state of sequence b in the workspace (zero between calls):
// word 0 counts the passes the sequence's blocks have published (each block
// bumps it once a pass), word 1 the blocks that are done, word 2 is set when a
// wait ran out, and words 4 + kMultiSplit * (pass & 1) + g hold block g's
// remainder mass of a pass (two sets: a block publishes pass p + 1 only after
// every block published pass p, which each did after reading pass p - 1).
__device__ __forceinline__ int* msync_of(const Params& P, int b) {
  return P.msync + (size_t)b * kMultiSyncWords;
}

// Every block of sequence b publishes, then waits (bounded) until all have
// published this pass.
__device__ void seq_sync(const Params& P, MultiShared& S, int b) {
  drain_stores();
  __syncthreads();
  if (threadIdx.x == 0) {
    int* ctr = msync_of(P, b);
    bump(ctr);
    const int want = kMultiSplit * (S.pass + 1);
    for (int spins = 0; obs_i(ctr) < want; ++spins) {
      if (spins >= P.spin_limit) {
        S.to = 1;
        break;
      }
      __builtin_amdgcn_s_sleep(2);
    }
    S.pass += 1;
  }
  __syncthreads();
}

// Block reductions and scan over the kMT threads (every thread gets the result).
__device__ __forceinline__ float mt_sum(MultiShared& S, float x) {
  x = wave_sum(x);
  __syncthreads();
  if ((threadIdx.x & (kWave - 1)) == 0) S.red[threadIdx.x / kWave] = x;
  __syncthreads();
  float a = 0.f;
#pragma unroll
  for (int k = 0; k < kMW; ++k) a += S.red[k];
  return a;
}
__device__ __forceinline__ float mt_incl_scan(MultiShared& S, float x, float& total) {
  const int lane = threadIdx.x & (kWave - 1), w = threadIdx.x / kWave;
  const float incl = wave_incl_scan(x);
  __syncthreads();
  if (lane == kWave - 1) S.red[w] = incl;
  __syncthreads();
  float base = 0.f;
  total = 0.f;
#pragma unroll
  for (int k = 0; k < kMW; ++k) {
    const float t = S.red[k];
    if (k < w) base += t;
    total += t;
  }
  return base + incl;
}
template <bool MIN>
__device__ __forceinline__ int mt_ext_i(MultiShared& S, int x) {
  x = MIN ? wave_min_i(x) : wave_max_i(x);
  __syncthreads();
  if ((threadIdx.x & (kWave - 1)) == 0) S.redi[threadIdx.x / kWave] = x;
  __syncthreads();
  int r = S.redi[0];
#pragma unroll
  for (int k = 1; k < kMW; ++k) r = MIN ? min(r, S.redi[k]) : max(r, S.redi[k]);
  return r;
}

// Law of the N ids of one vector at the current node: r = p, with each of the
// NR rejected candidates' q peeled off in turn, r <- max(0, r - q_k)/Z_k. With
// EXTRA, also d = max(0, r - q_extra) (the mass a rejection of that candidate
// leaves).
template <int DT, bool VEC, bool FILT, int NR, bool EXTRA>
__device__ __forceinline__ void law_of(const Params& P, const MultiShared& S,
                                       const typename Vec<DT, VEC>::Raw* rv, float* r, float* d) {
  using Vc = Vec<DT, VEC>;
  constexpr int N = Vc::N;
  const float c = P.c;
  float f[N];
  Vc::get(rv[0], f);
  const RowS p = S.p;
#pragma unroll
  for (int e = 0; e < N; ++e) r[e] = prob_of<FILT>(f[e], p, c);
#pragma unroll
  for (int k = 0; k < NR; ++k) {
    Vc::get(rv[1 + k], f);
    const RowS q = S.q[k];
    const float iz = S.iZ[k];
#pragma unroll
    for (int e = 0; e < N; ++e) r[e] = fmaxf(r[e] - prob_of<FILT>(f[e], q, c), 0.f) * iz;
  }
  if constexpr (EXTRA) {
    Vc::get(rv[1 + NR], f);
    const RowS xq = S.xq;
#pragma unroll
    for (int e = 0; e < N; ++e) d[e] = fmaxf(r[e] - prob_of<FILT>(f[e], xq, c), 0.f);
  }
}

// The rows of vector v at the current node: p, the NR rejected q's and (EXTRA)
// the candidate's q; zero vectors past the row's end.
template <int DT, bool VEC, int NR, bool EXTRA>
__device__ __forceinline__ void load_rows(const Params& P, const MultiShared& S, int v,
                                          typename Vec<DT, VEC>::Raw* rv) {
  using Vc = Vec<DT, VEC>;
  constexpr int R = 1 + NR + (EXTRA ? 1 : 0);
  const bool in = v < P.nvec;
#pragma unroll
  for (int k = 0; k < R; ++k) {
    const void* base = k == 0 ? P.target : P.draft;
    const int row = k == 0 ? S.prow : (k <= NR ? S.qrow[k - 1] : S.xrow);
    rv[k] = in ? Vc::load(base, (size_t)row * P.V, v) : typename Vc::Raw{};
  }
}

// One pass over this block's tiles of the vocabulary (whole block). With
// EXTRA it returns the block's sum of max(0, r - q_extra) (its part of the
// next remainder's mass). Otherwise it leaves per-tile sums of r in S.tsum
// (one wave sum per tile and wave) and returns 0.
template <int DT, bool VEC, bool FILT, int NR, bool EXTRA>
__device__ float vocab_pass(const Params& P, MultiShared& S) {
  using Vc = Vec<DT, VEC>;
  constexpr int N = Vc::N;
  using Raw = typename Vc::Raw;
  constexpr int R = 1 + NR + (EXTRA ? 1 : 0);
  constexpr int NBT = multi_batch(R);
  const int tid = threadIdx.x;
  const int lane = tid & (kWave - 1), wave = tid / kWave;
  const int tb = S.tb, te = S.te;
  float total = 0.f;
  for (int t0 = tb; t0 < te; t0 += NBT) {
    Raw rv[NBT][R];
#pragma unroll
    for (int i = 0; i < NBT; ++i)
      load_rows<DT, VEC, NR, EXTRA>(P, S, t0 + i < te ? (t0 + i) * kMTile + tid : P.nvec, rv[i]);
#pragma unroll
    for (int i = 0; i < NBT; ++i) {
      const int v = (t0 + i) * kMTile + tid;
      float r[N], d[N];
      law_of<DT, VEC, FILT, NR, EXTRA>(P, S, rv[i], r, d);
      float w = 0.f;
      if (t0 + i < te && v < P.nvec) {
#pragma unroll
        for (int e = 0; e < N; ++e) w += EXTRA ? d[e] : r[e];
      }
      if constexpr (EXTRA) {
        total += w;
      } else if (t0 + i < te) {
        const float ws = wave_sum(w);
        if (lane == 0) S.tsum[t0 + i][wave] = ws;
      }
    }
  }
  if constexpr (!EXTRA) {
    __syncthreads();
    return 0.f;
  } else {
    return mt_sum(S, total);
  }
}

// The mass max(0, r - q_candidate) summed over the vocabulary: each block's
// part, published, then the parts added in block order (the same sum in every
// block of the sequence).
template <int DT, bool VEC, bool FILT>
__device__ float remainder_part(const Params& P, MultiShared& S) {
  switch (S.nrej) {
    case 0: return vocab_pass<DT, VEC, FILT, 0, true>(P, S);
    case 1: return vocab_pass<DT, VEC, FILT, 1, true>(P, S);
    case 2: return vocab_pass<DT, VEC, FILT, 2, true>(P, S);
    default: return vocab_pass<DT, VEC, FILT, SV_MAX_CHAINS - 1, true>(P, S);
  }
}
template <int DT, bool VEC, bool FILT>
__device__ __forceinline__ float remainder_mass(const Params& P, MultiShared& S, int b, int g) {
  const float part = remainder_part<DT, VEC, FILT>(P, S);
  float* parts = reinterpret_cast<float*>(msync_of(P, b) + 4 + kMultiSplit * (S.pass & 1));
  if (threadIdx.x == 0) pub_f(parts + g, part);
  seq_sync(P, S, b);
  float z = 0.f;
#pragma unroll
  for (int k = 0; k < kMultiSplit; ++k) z += obs_f(parts + k);
  return z;
}

// Inverse CDF of the current law with uniform u (whole block): the smallest
// id whose cumulative weight in ascending id order exceeds u * Z; if rounding
// leaves none, the last id with positive weight.
template <int DT, bool VEC, bool FILT, int NR>
__device__ int draw_law_n(const Params& P, MultiShared& S, float u, int b) {
  using Vc = Vec<DT, VEC>;
  constexpr int N = Vc::N;
  using Raw = typename Vc::Raw;
  const int tid = threadIdx.x;
  const int T = (P.nvec + kMTile - 1) / kMTile;
  vocab_pass<DT, VEC, FILT, NR, false>(P, S);
  // this block's tile totals to the sequence's list, then every tile's
  float* tiles = P.mtiles + (size_t)b * P.mtiles_stride;
  for (int t = S.tb + tid; t < S.te; t += kMT) {
    float s = 0.f;
#pragma unroll
    for (int w = 0; w < kMW; ++w) s += S.tsum[t][w];
    pub_f(tiles + t, s);
  }
  seq_sync(P, S, b);
  if (S.to) return -1;
  for (int t = tid; t < T; t += kMT) S.tsum[t][0] = obs_f(tiles + t);
  __syncthreads();
  if (tid == 0) {
    float z = 0.f;
    for (int t = 0; t < T; ++t) z += S.tsum[t][0];
    const float target = u * z;
    int ct = -1, last = -1;
    float run = 0.f, base = 0.f, lbase = 0.f;
    for (int t = 0; t < T; ++t) {
      const float s = S.tsum[t][0];
      if (ct < 0 && run + s > target) {
        ct = t;
        base = run;
      }
      if (s > 0.f) {
        last = t;
        lbase = run;
      }
      run += s;
    }
    if (ct < 0) {
      ct = last < 0 ? 0 : last;
      base = last < 0 ? 0.f : lbase;
    }
    S.ct = ct;
    S.base = base;
    S.target = target;
  }
  __syncthreads();
  const int ct = S.ct;
  if (ct < S.tb || ct >= S.te) return -1;  // another block of the sequence picks
  const float base = S.base, target = S.target;
  const int v = ct * kMTile + tid;
  Raw rv[1 + NR];
  load_rows<DT, VEC, NR, false>(P, S, v, rv);
  float r[N], d[N], w[N];
  law_of<DT, VEC, FILT, NR, false>(P, S, rv, r, d);
  float acc = 0.f;
#pragma unroll
  for (int e = 0; e < N; ++e) {
    acc += (v < P.nvec) ? r[e] : 0.f;
    w[e] = acc;
  }
  float tot;
  const float excl = base + (mt_incl_scan(S, acc, tot) - acc);
  int cand = INT_MAX, lastpos = -1;
  float prev = 0.f;
#pragma unroll
  for (int e = 0; e < N; ++e) {
    if (cand == INT_MAX && excl + w[e] > target) cand = v * N + e;
    if (w[e] > prev) lastpos = v * N + e;
    prev = w[e];
  }
  int tok = mt_ext_i<true>(S, cand);
  if (tok == INT_MAX) tok = mt_ext_i<false>(S, lastpos);
  if (tok < 0) tok = ct * kMTile * N;
  return tok;
}

// The drawn token in the block whose tiles hold the crossing, -1 in the others.
template <int DT, bool VEC, bool FILT>
__device__ __forceinline__ int draw_law(const Params& P, MultiShared& S, float u, int b) {
  switch (S.nrej) {
    case 0: return draw_law_n<DT, VEC, FILT, 0>(P, S, u, b);
    case 1: return draw_law_n<DT, VEC, FILT, 1>(P, S, u, b);
    case 2: return draw_law_n<DT, VEC, FILT, 2>(P, S, u, b);
    case 3: return draw_law_n<DT, VEC, FILT, 3>(P, S, u, b);
    default: return draw_law_n<DT, VEC, FILT, SV_MAX_CHAINS>(P, S, u, b);
  }
}

// One sequence (one block): see the file comment.
template <int DT, bool VEC, bool FILT>
__global__ __launch_bounds__(kMT, 1) void k_multi(const Params P) {
  __shared__ MultiShared S;
  __shared__ int s_last;
  const int tid = threadIdx.x;
  // kMultiSplit consecutive blocks walk sequence b, block g on the g-th
  // contiguous range of the vocabulary's tiles
  const int b = blockIdx.x / kMultiSplit, g = blockIdx.x % kMultiSplit;
  const int M = P.M, K = P.K;
  const float c = P.c;
  const int t_out = b * (K + 1);
  if (tid == 0) {
    const int T = (P.nvec + kMTile - 1) / kMTile;
    S.tb = g * T / kMultiSplit;
    S.te = (g + 1) * T / kMultiSplit;
    S.pass = 0;
    S.to = 0;
  }
  // draft ids of every chain: any outside [0, V) makes the sequence invalid
  int bad = 0;
  for (int k = tid; k < M * K; k += kMT) {
    const int x = P.tokens[(size_t)b * M * K + k];
    bad |= !(x >= 0 && x < P.V);
  }
  const int badtok = __syncthreads_or(bad);
  int live = (1 << M) - 1;
  int n = -1, code = badtok ? SV_SEQ_BAD_TOKEN : 0, tok = -1, lead = 0;
  // Greedy (temperature 0): the target law is a point mass at the argmax of
  // the lowest live chain's row (lowest id on ties); the first live chain
  // proposing it is accepted, and when none does it is emitted. No pass over
  // the vocabulary, so every block of the sequence takes the same steps
  // without exchanging anything; block 0 writes the outputs.
  for (int j = 0; P.all_greedy && j <= K && code == 0 && n < 0; ++j) {
    lead = __builtin_ctz((unsigned)live);
    if (tid == 0) {
      const int prow = (b * M + lead) * (K + 1) + j;
      float v = kNegInf;
      int am = INT_MAX, bad = 0;
      merge_greedy(P.slots + unit_of(P, true, prow) * P.chunks, P.chunks, v, am, bad);
      S.pok = !bad && v != kNegInf;
      S.tok = am;
    }
    __syncthreads();
    if (!S.pok) {
      code = SV_SEQ_BAD_ROW;
      break;
    }
    const int a = S.tok;
    __syncthreads();  // every thread has read S before thread 0 writes it again
    int keep = 0;
    if (j < K)
      for (int m = 0; m < M; ++m)
        if ((live & (1 << m)) && P.tokens[((size_t)b * M + m) * K + j] == a) keep |= 1 << m;
    if (keep == 0) {
      tok = g == 0 ? a : -1;
      n = j;
      break;
    }
    if (tid == 0 && g == 0) pub_i(P.out_tokens + t_out + j, a);
    live = keep;
  }
  for (int j = 0; !P.all_greedy && j <= K && code == 0 && n < 0; ++j) {
    lead = __builtin_ctz((unsigned)live);
    const int s_lead = b * M + lead;  // chain lead as a sequence of the statistics pass
    if (tid == 0) {
      S.prow = s_lead * (K + 1) + j;
      S.p = merged_row(P, unit_of(P, true, S.prow));
      S.nrej = 0;
      S.pok = S.p.ok;
    }
    __syncthreads();
    if (!S.pok) {
      code = SV_SEQ_BAD_ROW;
      break;
    }
    const float* ub = P.uniforms + ((size_t)b * (K + 1) + j) * (M + 1);
    if (j == K) {  // bonus: draw from p_K of the lowest live chain
      tok = draw_law<DT, VEC, FILT>(P, S, ub[M], b);
      n = K;
      break;
    }
    int accepted = -1;
    for (int m = 0; m < M; ++m) {
      if (!(live & (1 << m))) continue;
      // thread 0 tests chain m's candidate against the current law
      if (tid == 0) {
        const int s = b * M + m;
        const int drow = s * K + j;
        const RowS q = merged_row(P, unit_of(P, false, drow));
        S.xrow = drow;
        S.xq = q;
        if (!q.ok) {
          S.act = 4;
        } else {
          const int x = P.tokens[(size_t)s * K + j];
          float r = prob_of<true>(load_elem<DT>(P.target, (size_t)S.prow * P.V + x), S.p, c);
          for (int k = 0; k < S.nrej; ++k)
            r = fmaxf(r - prob_of<true>(load_elem<DT>(P.draft, (size_t)S.qrow[k] * P.V + x),
                                        S.q[k], c), 0.f) * S.iZ[k];
          const float qx = prob_of<true>(load_elem<DT>(P.draft, (size_t)drow * P.V + x), q, c);
          // r/q with q(x) = 0 < r(x) accepting and r(x) = q(x) = 0 rejecting
          const float ratio = r / qx;
          S.act = ub[m] < ratio ? 1 : 2;
        }
      }
      __syncthreads();
      const int act = S.act;
      if (act == 4) {
        code = SV_SEQ_BAD_ROW;
        break;
      }
      if (act == 1) {
        accepted = m;
        break;
      }
      // rejected: the mass the remainder keeps, then the remainder is the law
      const float z = remainder_mass<DT, VEC, FILT>(P, S, b, g);
      if (S.to) break;
      if (tid == 0 && z > 0.f) {
        // a mass that rounds to zero keeps the current law
        S.q[S.nrej] = S.xq;
        S.qrow[S.nrej] = S.xrow;
        S.iZ[S.nrej] = 1.0f / z;
        S.nrej += 1;
      }
      __syncthreads();
    }
    if (code != 0 || S.to) break;
    if (accepted < 0) {
      tok = draw_law<DT, VEC, FILT>(P, S, ub[M], b);
      n = j;
      break;
    }
    // the accepted token; the chains that proposed it stay alive
    const int t = P.tokens[((size_t)b * M + accepted) * K + j];
    if (tid == 0 && g == 0) pub_i(P.out_tokens + t_out + j, t);
    int keep = 0;
    for (int m = 0; m < M; ++m)
      if ((live & (1 << m)) && P.tokens[((size_t)b * M + m) * K + j] == t) keep |= 1 << m;
    live = keep;
    __syncthreads();
  }
  // outputs: block 0 wrote the prefix as it was accepted and writes the
  // padding, n and the chain holding the prefix; the block whose tiles held
  // the draw's crossing writes the drawn token
  const bool timed = S.to != 0;
  if (!timed) {
    if (code != 0) {
      if (g == 0) {
        for (int k = tid; k <= K; k += kMT) P.out_tokens[t_out + k] = -1;
        if (tid == 0) {
          P.num_accepted[b] = code;
          if (P.out_chain) P.out_chain[b] = -1;
        }
      }
    } else {
      if (g == 0) {
        for (int k = tid + n + 1; k <= K; k += kMT) P.out_tokens[t_out + k] = -1;
        if (tid == 0) {
          P.num_accepted[b] = n;
          if (P.out_chain) P.out_chain[b] = lead;
        }
      }
      if (tok >= 0 && tid == 0) P.out_tokens[t_out + n] = tok;
    }
  }
  // Every block counts itself done; the last one reports a timed-out wait of
  // any of them and returns the sequence's workspace entries to zero.
  int* sy = msync_of(P, b);
  if (timed && tid == 0) raise_flag(sy + 2, 1);
  drain_stores();
  __syncthreads();
  if (tid == 0) s_last = bump(sy + 1) == kMultiSplit - 1;
  __syncthreads();
  if (!s_last) return;
  if (obs_i(sy + 2) != 0) {
    for (int k = tid; k <= K; k += kMT) P.out_tokens[t_out + k] = -1;
    if (tid == 0) {
      P.num_accepted[b] = SV_SEQ_SYNC_TIMEOUT;
      if (P.out_chain) P.out_chain[b] = -1;
    }
  }
  for (int k = tid; k < kMultiSyncWords; k += kMT) pub_i(sy + k, 0);
  const int T = (P.nvec + kMTile - 1) / kMTile;
  for (int t = tid; t < T; t += kMT) pub_f(P.mtiles + (size_t)b * P.mtiles_stride + t, 0.f);
  // the statistics pass's partials (and with filters the cut pass's row
  // results) of this sequence's rows back to zero
  const int C = P.chunks;
  const long long d_units = (long long)M * K * C, t_units = (long long)M * (K + 1) * C;
  for (long long k = tid; k < d_units + t_units; k += kMT) {
    const bool tgt = k >= d_units;
    const long long kk = tgt ? k - d_units : k;
    const long long row = (tgt ? (long long)b * M * (K + 1) : (long long)b * M * K) + kk / C;
    P.slots[unit_of(P, tgt, (int)row) * C + kk % C] = 0ull;
  }
  if (P.filt) {
    const int nd = M * K, nt = M * (K + 1);
    for (int k = tid; k < nd + nt; k += kMT) {
      const bool tgt = k >= nd;
      const int row = tgt ? b * nt + (k - nd) : b * nd + k;
      P.rowres[unit_of(P, tgt, row)] = RowRes{0.f, 0.f, 0.f, 0};
    }
  }
}

template <int DT>
void launch_multi_dt(bool vec, const Params& P, dim3 grid, dim3 block, hipStream_t s) {
  if (P.filt) {
    if (vec) hipLaunchKernelGGL((k_multi<DT, true, true>), grid, block, 0, s, P);
    else hipLaunchKernelGGL((k_multi<DT, false, true>), grid, block, 0, s, P);
  } else {
    if (vec) hipLaunchKernelGGL((k_multi<DT, true, false>), grid, block, 0, s, P);
    else hipLaunchKernelGGL((k_multi<DT, false, false>), grid, block, 0, s, P);
  }
}

}  // namespace

hipError_t launch_multi(int dtype, bool vec, const Params& P, hipStream_t s) {
  const dim3 grid((unsigned)(P.B / P.M * kMultiSplit)), block(kMT);
  switch (dtype) {
    case SV_F32: launch_multi_dt<SV_F32>(vec, P, grid, block, s); break;
    case SV_F16: launch_multi_dt<SV_F16>(vec, P, grid, block, s); break;
    default: launch_multi_dt<SV_BF16>(vec, P, grid, block, s);
  }
  return hipGetLastError();
}

}  // namespace sv
