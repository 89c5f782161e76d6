// Verification from LM-head hidden states for gfx950: the logits l = h W^T of
// every draft and target row are formed on the matrix cores (bf16 operands,
// fp32 accumulation), reduced in the GEMM's epilogue to per-row softmax
// partials, and stored as fp32 for the final draw, which reads two rows per
// sequence (p_n, and q_n for a residual).
//
//   k_lm_stats        draft rows, then target rows: per (row, 384-id vocab
//                     tile) the packed (max, sum of 2^(l*c - R)) partial, the
//                     logit at the row's token, and the logits themselves
//   k_lm_merge        per row: the vocabulary tiles' partials merged into one
//                     (and returned to zero)
//   k_draw            the decision, the outputs, and the inverse-CDF draw over
//                     the stored rows (the same kernel as the logit path)
//
// Storing every row costs the statistics GEMM about 95 us at B = 64, K = 8,
// V = 128256 (558 MB of writes beside its loads); forming the two draw rows of
// each sequence again instead streamed both weights a second time (1.58 GB,
// 303-336 us).
//
// Greedy verification (temperature 0) reads no draft rows: k_lm_stats<true>
// runs on the target rows alone, with per tile the packed (max, argmax with
// the lowest id on ties, NaN / +inf seen) partial of the logit path's greedy
// rows; k_lm_merge_am merges them, and k_draw decides and writes the outputs
// (the correction or bonus token is the argmax, so no row is formed again).
//
// Pages (by title, section): Hung-yi Lee lecture-16 notes (the target model
// scores every drafted position in one forward pass; the logits are its last
// layer's output); aivaro.ru answer 289 "Как работает speculative decoding на
// уровне логитов, а не токенов?" s.8 (the memory the draft and target logits
// take up), s.6 and s.9 (ratio test, residual).
#include <utility>

#include "sv_rows.h"

namespace sv {

namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

constexpr int kXcds = 8;  // blocks are dealt round-robin to the eight XCDs

struct LmGemm {
  const uint16_t* H;   // hidden rows, bf16 bits, row stride D
  const uint16_t* W;   // LM-head weight [V, D], bf16 bits
  int M, D, V, NT, MT;  // rows, hidden size, vocabulary, vocabulary tiles, row tiles
  // statistics epilogue
  unsigned long long* part;  // [(unit0 + m) * NT + vt]
  float* tok_logits;         // [unit0 + m]
  long long unit0;
  int K;                     // drafts per sequence (dense)
  int target;                // 1: rows are target rows, their token is x_i for i < K
  const int32_t* tokens;
  float c;
  float* out;                // logits: row m to out[m * V + v] (null: not stored)
};

// Two GEMMs in one launch (the draft's and the target's): blocks below n0
// run the first, the rest the second. n0 is a multiple of eight, so both keep
// the XCD-aware block order.
struct LmPair {
  LmGemm g[2];
  int n0;
};

// ---------------------------------------------------------------------------
// Statistics GEMM (k_lm_stats). Block tile: 192 rows x 384 vocabulary ids, 12
// waves in a 2 x 6 arrangement, each a 96 x 64 sub-tile of 3 x 2 32 x 32 MFMA
// tiles; 64 hidden elements per step. Both operand tiles of a step ([hidden
// rows; weight rows], 128 bytes a row) are filled by direct global -> LDS
// loads into one of two stages while the MFMAs read the other, so no operand
// passes through registers before the MFMA reads it.
//
// Why this shape: every 16-byte operand chunk the compute units fetch comes
// from L2 (or further), and that stream, not the matrix cores, set the pace of
// the earlier 128 x 256 tile (7.6 GB fetched a call at the target workload,
// about 450 us at the rate the fetch path sustains). Per call the fetch is
// (hidden bytes) x (vocabulary tiles) + (weight bytes) x (row tiles): 192 rows
// divide 576 target rows into three tiles and 384 ids divide V = 128256 into
// 334, which brings it to 4.7 GB. Twelve waves (three per SIMD) hide the LDS
// reads of one wave behind the MFMAs of the others.
constexpr int kStBM = 192, kStBN = 384, kStBK = 64;
constexpr int kStWM = 2, kStWN = 6;                          // waves along rows, ids
constexpr int kStTM = 3, kStTN = 2;                          // MFMA tiles per wave
constexpr int kStWaves = kStWM * kStWN;
constexpr int kStThreads = kStWaves * kWave;
constexpr int kStRowBytes = kStBK * 2;                       // one operand row of a step
constexpr int kStStageBytes = (kStBM + kStBN) * kStRowBytes;  // 72 KB
constexpr int kStDma = kStStageBytes / 1024 / kStWaves;      // 1 KB loads per wave and stage
constexpr int kStSlots = kStBN / 64;                          // 64-id slices of a tile row
constexpr int kStEp = 64 + 4;                                 // epilogue staging row (floats)
static_assert(kStBM == kStWM * kStTM * 32 && kStBN == kStWN * kStTN * 32 && kStTN == 2,
              "each wave covers one 64-id slice of the tile");
static_assert(kStStageBytes % (1024 * kStWaves) == 0, "the loads split evenly over the waves");
static_assert(kStWaves * 32 * kStEp * 4 <= 2 * kStStageBytes, "epilogue staging fits the stages");

// Read by the loads of hidden elements past D (a step that D ends inside).
__device__ __align__(16) const uint16_t kLmZeros[8] = {0, 0, 0, 0, 0, 0, 0, 0};

typedef __attribute__((address_space(3))) void* lds_void_ptr;
typedef __attribute__((address_space(1))) void* global_void_ptr;

// s_waitcnt immediate: vector memory count 0, the other counters unconstrained
constexpr int kWaitVm0 = (7 << 4) | (15 << 8);

// One block: a 192 x 384 tile of logits, reduced per row and 64-id slice in
// the epilogue and merged into one partial per (row, tile). The block order is
// XCD-aware: block g runs on XCD g % 8, and the row tiles of one vocabulary
// tile are consecutive blocks of one XCD, so its weight tile is fetched into
// that XCD's L2 once and read from there by the other row tiles. GREEDY:
// (max, argmax, NaN/+inf) partials instead of (max, sum).
template <bool GREEDY>
__global__ __launch_bounds__(kStThreads, 3) void k_lm_stats(const LmPair PR) {
  const bool second = (int)blockIdx.x >= PR.n0;
  const LmGemm& G = PR.g[second ? 1 : 0];
  // Two operand stages (after the main loop the epilogue stages its slices
  // there), then the per-slot partials and the rows' tokens. One LDS array:
  // with several, the compiler waits for the loads into one stage before
  // every read of the other.
  __shared__ __align__(16) unsigned char s_lds[2 * kStStageBytes + (2 * kStSlots + 1) * kStBM * 4];
  unsigned char* const s_op = s_lds;
  float (*const s_pm)[kStBM] = reinterpret_cast<float (*)[kStBM]>(s_lds + 2 * kStStageBytes);
  // greedy: the argmax, bit 31 NaN or +inf seen
  float (*const s_ps)[kStBM] = s_pm + kStSlots;
  int* const s_tok = reinterpret_cast<int*>(s_ps + kStSlots);
  const int tid = threadIdx.x;
  const int lane = tid & (kWave - 1);
  const int wave = tid / kWave;
  const int wm = wave % kStWM, wn = wave / kStWM;
  const int g = (int)blockIdx.x - (second ? PR.n0 : 0);
  const int idx = g / kXcds;
  const int vt = (idx / G.MT) * kXcds + g % kXcds;
  const int mt = idx % G.MT;
  if (vt >= G.NT) return;
  const int m0 = mt * kStBM, v0 = vt * kStBN;

  // Load i of this wave fills 1 KB q = wave + kStWaves * i of a stage: tile
  // rows 8q .. 8q + 7 (hidden rows first, then weight rows); lane l the row
  // 8q + l / 8 and 16-byte slot l % 8, which holds chunk (l % 8) ^ swz(row)
  // of the step. gfx950's LDS serves a 16-byte read of 16 lanes at once from
  // 64 banks; with 128-byte rows, rows r and r + 1 sit on the two halves of
  // the banks, so swz(r) = (r / 2) % 8 gives the 16 rows that 16 lanes read
  // at one chunk column 16 distinct bank groups (r % 8 would put rows r and
  // r + 8 on the same ones: 2-way conflicts on every read). Rows past M or V
  // repeat the last row; their results are never used.
  const uint16_t* src[kStDma];
  int kch[kStDma];  // first hidden element of this lane's chunk within a step
#pragma unroll
  for (int i = 0; i < kStDma; ++i) {
    const int q = wave + kStWaves * i;
    const int r = q * 8 + (lane >> 3);
    const int cg = (lane & 7) ^ ((r >> 1) & 7);
    const uint16_t* row;
    if (r < kStBM) {
      const int m = min(m0 + r, G.M - 1);
      row = G.H + (size_t)m * G.D;
    } else {
      const int v = min(v0 + r - kStBM, G.V - 1);
      row = G.W + (size_t)v * G.D;
    }
    kch[i] = cg * 8;
    src[i] = row + kch[i];
  }
  const int nsteps = (G.D + kStBK - 1) / kStBK;
  // the loads of step st into a stage; chunks past D read zeros. Kept
  // free of branches: the compiler then tracks these loads precisely and does
  // not wait for them before the MFMAs' LDS reads of the other stage.
  auto issue = [&](int st, int stage) {
    unsigned char* base = s_op + stage * kStStageBytes + wave * 1024;
    const int k0 = st * kStBK;
#pragma unroll
    for (int i = 0; i < kStDma; ++i) {
      const uint16_t* p = (k0 + kch[i] < G.D) ? src[i] + k0 : kLmZeros;
      __builtin_amdgcn_global_load_lds((global_void_ptr)p,
                                       (lds_void_ptr)(base + i * kStWaves * 1024), 16, 0, 0);
    }
  };

  f32x16 acc[kStTM][kStTN];
#pragma unroll
  for (int a = 0; a < kStTM; ++a)
#pragma unroll
    for (int b = 0; b < kStTN; ++b)
#pragma unroll
      for (int i = 0; i < 16; ++i) acc[a][b][i] = 0.0f;

  issue(0, 0);
  for (int t = 0; t < nsteps; ++t) {
    // this wave's loads of step t have landed; the barrier makes every wave's
    // visible and ends every wave's reads of step t - 1, whose stage the
    // loads of step t + 1 then fill (the last step repeats its own loads into
    // the other stage, which nothing reads)
    __builtin_amdgcn_s_waitcnt(kWaitVm0);
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
    issue(min(t + 1, nsteps - 1), (t + 1) & 1);
    const unsigned char* base = s_op + (t & 1) * kStStageBytes;
    // lane l reads row l % 32 of each 32 x 32 tile, chunk 2 ks + l / 32 of
    // the step (8 consecutive hidden elements)
    bf16x8 af[2][kStTM], bfr[2][kStTN];
    auto rd = [&](int ks, int sl) {
      const int cg = ks * 2 + (lane >> 5);
#pragma unroll
      for (int a = 0; a < kStTM; ++a) {
        const int r = wm * kStTM * 32 + a * 32 + (lane & 31);
        af[sl][a] = *reinterpret_cast<const bf16x8*>(base + r * kStRowBytes + ((cg ^ ((r >> 1) & 7)) * 16));
      }
#pragma unroll
      for (int b = 0; b < kStTN; ++b) {
        const int r = kStBM + wn * kStTN * 32 + b * 32 + (lane & 31);
        bfr[sl][b] = *reinterpret_cast<const bf16x8*>(base + r * kStRowBytes + ((cg ^ ((r >> 1) & 7)) * 16));
      }
    };
    rd(0, 0);
#pragma unroll
    for (int ks = 0; ks < kStBK / 16; ++ks) {
      if (ks + 1 < kStBK / 16) rd(ks + 1, (ks + 1) & 1);
#pragma unroll
      for (int a = 0; a < kStTM; ++a)
#pragma unroll
        for (int b = 0; b < kStTN; ++b)
          acc[a][b] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[ks & 1][a], bfr[ks & 1][b],
                                                               acc[a][b], 0, 0, 0);
    }
    // the first substep's reads, then one read of the next substep after each MFMA
    __builtin_amdgcn_sched_group_barrier(0x100, kStTM + kStTN, 0);
#pragma unroll
    for (int ks = 0; ks < kStBK / 16; ++ks) {
      if (ks + 1 < kStBK / 16) {
#pragma unroll
        for (int i = 0; i < kStTM + kStTN; ++i) {
          __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
          __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
        }
        __builtin_amdgcn_sched_group_barrier(0x008, kStTM * kStTN - (kStTM + kStTN), 0);
      } else {
        __builtin_amdgcn_sched_group_barrier(0x008, kStTM * kStTN, 0);
      }
    }
  }

  // Element i of tile (a, b) in lane l: row wm*96 + a*32 + 8*(i/4) + 4*(l/32)
  // + i%4, vocabulary id v0 + wn*64 + b*32 + l%32.
  // The logits themselves: the sampling call's draw reads two rows per
  // sequence, and spec_verify_lmhead_diag returns them. Non-temporal stores:
  // nothing reads them again before the draw, so they need not displace the
  // operands in L2.
  if (G.out != nullptr) {
#pragma unroll
    for (int a = 0; a < kStTM; ++a) {
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const int m = m0 + wm * kStTM * 32 + a * 32 + 8 * (i >> 2) + 4 * (lane >> 5) + (i & 3);
        if (m >= G.M) continue;
        float* orow = G.out + (size_t)m * G.V;
#pragma unroll
        for (int b = 0; b < kStTN; ++b) {
          const int v = v0 + wn * kStTN * 32 + b * 32 + (lane & 31);
          if (v < G.V) __builtin_nontemporal_store(acc[a][b][i], orow + v);
        }
      }
    }
  }
  if (tid < kStBM) {
    const int m = m0 + tid;
    int tok = -1;
    if (m < G.M) {
      if (!G.target) {
        tok = G.tokens[m];
      } else {
        const int i = m % (G.K + 1);
        if (i < G.K) tok = G.tokens[(m / (G.K + 1)) * G.K + i];
      }
    }
    s_tok[tid] = tok;
  }
  // Each wave stages one 32 x 64 slice of its sub-tile at a time in LDS
  // (row-major, 4 floats of padding per row), then lane l reduces half of
  // row l / 2 (32 ids) and pairs with lane l ^ 1 for the slice's 64 ids.
  // Slot wn of s_pm / s_ps holds each row's partial of the wave's slice.
  // The last step's repeated loads land before any wave stages a slice.
  __builtin_amdgcn_s_waitcnt(kWaitVm0);
  float* const E = reinterpret_cast<float*>(s_op) + wave * 32 * kStEp;
  const float c = G.c;
  const int r = lane >> 1, h = (lane & 1) * 32;
  const int cb = v0 + wn * 64 + h;  // first id of this lane's half row
#pragma unroll
  for (int a = 0; a < kStTM; ++a) {
    __syncthreads();  // the operand stages, or the previous slice, are read
#pragma unroll
    for (int b = 0; b < kStTN; ++b)
#pragma unroll
      for (int i = 0; i < 16; ++i)
        E[(8 * (i >> 2) + 4 * (lane >> 5) + (i & 3)) * kStEp + b * 32 + (lane & 31)] = acc[a][b][i];
    __syncthreads();
    float x[32];
#pragma unroll
    for (int j = 0; j < 32; j += 4) {
      const float4 t4 = *reinterpret_cast<const float4*>(&E[r * kStEp + h + j]);
      x[j] = t4.x;
      x[j + 1] = t4.y;
      x[j + 2] = t4.z;
      x[j + 3] = t4.w;
    }
    const int rl = wm * kStTM * 32 + a * 32 + r;
    if constexpr (GREEDY) {
      // the largest logit of the 32 ids (NaN never wins), its lowest id
      // (none while every value is -inf) and whether any is NaN or +inf,
      // then with lane l ^ 1, the other half of the slice's 64 ids
      float mx = kNegInf;
      int bd = 0;
#pragma unroll
      for (int j = 0; j < 32; ++j) {
        if (cb + j >= G.V) x[j] = kNegInf;
        bd |= is_nan_or_posinf(x[j]) ? 1 : 0;
        mx = fmaxf(mx, x[j]);
      }
      int jm = 32;
#pragma unroll
      for (int j = 31; j >= 0; --j) jm = (x[j] == mx) ? j : jm;
      int ai = (mx > kNegInf) ? cb + jm : INT_MAX;
      const float omx = dpp_f<0xB1>(mx);  // quad_perm [1,0,3,2]: lane l ^ 1
      const int oai = dpp_i<0xB1>(ai);
      bd |= dpp_i<0xB1>(bd);
      argmax_merge(mx, ai, omx, oai);
      if ((lane & 1) == 0) {
        s_pm[wn][rl] = mx;
        s_ps[wn][rl] = __uint_as_float((unsigned)ai | ((unsigned)bd << 31));
      }
    } else {
      const int tok = s_tok[rl];
      if (tok >= cb && tok < cb + 32) G.tok_logits[G.unit0 + m0 + rl] = E[r * kStEp + h + (tok - cb)];
      float mx = kNegInf;
#pragma unroll
      for (int j = 0; j < 32; ++j) {
        if (cb + j >= G.V) x[j] = kNegInf;
        mx = fmaxf(mx, x[j]);
      }
      mx = fmaxf(mx, dpp_f<0xB1>(mx));  // quad_perm [1,0,3,2]: lane l ^ 1
      const float R = ref_of(mx, c);
      float sm = 0.0f;
#pragma unroll
      for (int j = 0; j < 32; ++j) sm += fast_exp2(fmaf(x[j], c, -R));
      sm += dpp_f<0xB1>(sm);
      if ((lane & 1) == 0) {
        s_pm[wn][rl] = mx;
        s_ps[wn][rl] = sm;
      }
    }
  }
  __syncthreads();
  if (tid < kStBM && m0 + tid < G.M) {
    if constexpr (GREEDY) {
      // the slices in increasing id order: the strict compare keeps the first maximum
      float mm = s_pm[0][tid];
      const unsigned p0 = __float_as_uint(s_ps[0][tid]);
      int ai = (int)(p0 & 0x7fffffffu), bd = (int)(p0 >> 31);
#pragma unroll
      for (int q = 1; q < kStSlots; ++q) {
        const unsigned pq = __float_as_uint(s_ps[q][tid]);
        argmax_merge(mm, ai, s_pm[q][tid], (int)(pq & 0x7fffffffu));
        bd |= (int)(pq >> 31);
      }
      G.part[(size_t)(G.unit0 + m0 + tid) * G.NT + vt] = pack_am(mm, ai, bd);
    } else {
      float mm = s_pm[0][tid], ss = s_ps[0][tid];
#pragma unroll
      for (int q = 1; q < kStSlots; ++q) merge_ms(mm, ss, s_pm[q][tid], s_ps[q][tid], c);
      G.part[(size_t)(G.unit0 + m0 + tid) * G.NT + vt] = pack_ms(mm, ss);
    }
  }
}

// Per statistics unit: its vocabulary tiles' partials merged into one (a
// fixed tree over the block: each thread its run of tiles in order, then the
// wave and block merges), stored as the unit's only chunk; the tiles' partials
// go back to zero.
__global__ __launch_bounds__(kThreads) void k_lm_merge(const unsigned long long* part0,
                                                        unsigned long long* slots, int NT,
                                                        float c) {
  __shared__ float s_m[kThreads / kWave], s_s[kThreads / kWave];
  const long long u = blockIdx.x;
  unsigned long long* part = const_cast<unsigned long long*>(part0) + u * NT;
  const int tid = threadIdx.x;
  const int per = (NT + kThreads - 1) / kThreads;
  float m = kNegInf, s = 0.0f;
  for (int k = tid * per; k < min(NT, (tid + 1) * per); ++k) {
    float om, os;
    unpack_ms(part[k], om, os);
    merge_ms(m, s, om, os, c);
    part[k] = 0ull;
  }
  wave_reduce_ms(m, s, c);
  if ((tid & (kWave - 1)) == 0) {
    s_m[tid / kWave] = m;
    s_s[tid / kWave] = s;
  }
  __syncthreads();
  if (tid == 0) {
    float mm = s_m[0], ss = s_s[0];
#pragma unroll
    for (int w = 1; w < kThreads / kWave; ++w) merge_ms(mm, ss, s_m[w], s_s[w], c);
    slots[u] = pack_ms(mm, ss);
  }
}

// Per greedy statistics unit (from unit0): its vocabulary tiles' (max,
// argmax, NaN/+inf) partials merged into one, the lowest id on ties, stored
// as the unit's only chunk; the tiles' partials go back to zero.
__global__ __launch_bounds__(kThreads) void k_lm_merge_am(const unsigned long long* part0,
                                                           unsigned long long* slots, int NT,
                                                           long long unit0) {
  __shared__ float s_v[kThreads / kWave];
  __shared__ int s_i[kThreads / kWave], s_b[kThreads / kWave];
  const long long u = unit0 + blockIdx.x;
  unsigned long long* part = const_cast<unsigned long long*>(part0) + u * NT;
  const int tid = threadIdx.x;
  const int per = (NT + kThreads - 1) / kThreads;
  float v = kNegInf;
  int i = INT_MAX, bad = 0;
  for (int k = tid * per; k < min(NT, (tid + 1) * per); ++k) {
    float ov;
    int oi, ob;
    unpack_am(part[k], ov, oi, ob);
    argmax_merge(v, i, ov, oi);
    bad |= ob;
    part[k] = 0ull;
  }
  wave_argmax(v, i, bad);
  if ((tid & (kWave - 1)) == 0) {
    s_v[tid / kWave] = v;
    s_i[tid / kWave] = i;
    s_b[tid / kWave] = bad;
  }
  __syncthreads();
  if (tid == 0) {
    float vv = s_v[0];
    int ii = s_i[0], bb = s_b[0];
#pragma unroll
    for (int w = 1; w < kThreads / kWave; ++w) {
      argmax_merge(vv, ii, s_v[w], s_i[w]);
      bb |= s_b[w];
    }
    slots[u] = pack_am(vv, ii, bb);
  }
}

size_t align_up(size_t x) { return (x + 255) / 256 * 256; }

// Workspace of the LM-head path:
//   draw_done[B], seq_flags[B]   counters and status bits of the draw
//   slots[units]                 merged row partials (one chunk per unit)
//   tiles[B * ntiles]            draw-weight tile sums
//   part[units * NT]             vocabulary-tile partials of the GEMM epilogue
//   tok[units]                   logits at the units' tokens
// all zero between calls, and at the tail of the caller's workspace
//   logits[units * V] fp32       every row's logits, draft rows first (rewritten
//                                by every sampling call; greedy calls leave it)
// Calls of any shape may share a workspace sized for the largest: every
// shape's zero regions start at the front and its logits end at the back, and
// neither reaches the other's.
struct LmPlan {
  size_t off_draw_done, off_seq_flags, off_slots, off_tiles, off_part, off_tok, zero_bytes,
      logits_bytes, total;
  int NT, nvec, dchunks, ntiles;
};

bool lm_plan(int B, int K, int V, LmPlan& L) {
  if (B < 0 || K < 0 || K > SV_MAX_K || V < 1 || V > (1 << 30)) return false;
  const long long units = (long long)B * K + (long long)B * (K + 1);
  if (units > INT_MAX) return false;
  L.NT = (V + kStBN - 1) / kStBN;
  const bool vec = V % 4 == 0;
  L.nvec = vec ? V / 4 : V;
  L.dchunks = (L.nvec + kDrawVecs - 1) / kDrawVecs;
  L.ntiles = L.dchunks * kTilesPerDraw;
  size_t off = 0;
  L.off_draw_done = off;
  off += align_up((size_t)B * 4);
  L.off_seq_flags = off;
  off += align_up((size_t)B * 4);
  L.off_slots = off;
  off += align_up((size_t)units * 8);
  L.off_tiles = off;
  off += align_up((size_t)B * L.ntiles * 4);
  L.off_part = off;
  off += align_up((size_t)units * L.NT * 8);
  L.off_tok = off;
  off += align_up((size_t)units * 4);
  L.zero_bytes = off;
  L.logits_bytes = align_up((size_t)units * (size_t)V * 4);
  L.total = off + L.logits_bytes;
  return true;
}

}  // namespace

}  // namespace sv

extern "C" size_t spec_verify_lmhead_workspace_bytes(int B, int K, int V) {
  sv::LmPlan L;
  if (!sv::lm_plan(B, K, V, L)) return 0;
  return L.total > 0 ? L.total : 256;
}

extern "C" size_t spec_verify_lmhead_zero_bytes(int B, int K, int V) {
  sv::LmPlan L;
  if (!sv::lm_plan(B, K, V, L)) return 0;
  return L.zero_bytes;
}

namespace {

int run_lmhead(const void* hidden_draft, const void* weight_draft, int d_draft,
               const void* hidden_target, const void* weight_target, int d_target,
               const int32_t* draft_tokens, const float* uniforms, int B, int K, int V,
               float temperature, int32_t* out_tokens, int32_t* num_accepted, void* workspace,
               size_t workspace_bytes, hipStream_t stream, hipEvent_t* stage_events,
               int n_stage_events, float* logits_draft, float* logits_target) {
  using namespace sv;
  if (B < 0 || K < 0 || K > SV_MAX_K || V < 1) return SV_EINVAL;
  if (!(temperature >= 0.0f) || __builtin_isinf(temperature)) return SV_EINVAL;
  // temperature 0: greedy verification, which reads no draft rows and no uniforms
  const bool greedy = temperature == 0.0f;
  if (d_target < 8 || d_target % 8 != 0 ||
      (!greedy && K > 0 && (d_draft < 8 || d_draft % 8 != 0)))
    return SV_EINVAL;
  if (B == 0) return SV_OK;
  if (hidden_target == nullptr || weight_target == nullptr || out_tokens == nullptr ||
      num_accepted == nullptr || (!greedy && uniforms == nullptr))
    return SV_EINVAL;
  if (K > 0 && (draft_tokens == nullptr ||
                (!greedy && (hidden_draft == nullptr || weight_draft == nullptr))))
    return SV_EINVAL;
  // the draw reads the stored rows, the caller's logits arrays among them, in
  // 16-byte vectors
  const void* ptrs[6] = {hidden_draft, weight_draft, hidden_target, weight_target, logits_draft,
                         logits_target};
  for (const void* p : ptrs)
    if (p != nullptr && ((uintptr_t)p & 15u) != 0) return SV_EINVAL;
  LmPlan L;
  if (!lm_plan(B, K, V, L)) return SV_EUNSUPPORTED;
  if (workspace == nullptr || ((uintptr_t)workspace % 256) != 0 || workspace_bytes < L.total)
    return SV_EWORKSPACE;
  const int total_draft = B * K;
  const int rows = B * (K + 1);
  const long long gemm_d = (long long)L.NT * ((total_draft + kStBM - 1) / kStBM);
  const long long gemm_t = (long long)L.NT * ((rows + kStBM - 1) / kStBM);
  if (gemm_t + kXcds * 4 > (long long)INT_MAX || gemm_d + kXcds * 4 > (long long)INT_MAX)
    return SV_EUNSUPPORTED;
  char* ws = static_cast<char*>(workspace);
  // every row's logits at the tail of the workspace (256-byte aligned), draft
  // rows first; rows the caller asked for (the diag entry point) go to the
  // caller's arrays instead, and the draw reads them there
  const size_t off_logits = (workspace_bytes - L.logits_bytes) / 256 * 256;
  if (off_logits < L.zero_bytes) return SV_EWORKSPACE;
  float* const ws_logits = reinterpret_cast<float*>(ws + off_logits);
  float* const ldraft = logits_draft != nullptr ? logits_draft : ws_logits;
  float* const ltarget =
      logits_target != nullptr ? logits_target : ws_logits + (size_t)total_draft * V;

  Params P{};
  P.draft = ldraft;
  P.target = ltarget;
  P.tokens = draft_tokens;
  P.uniforms = uniforms;
  P.cu = nullptr;
  P.greedy = nullptr;
  P.B = B;
  P.K = K;
  P.V = V;
  P.total_draft = total_draft;
  P.rows = rows;
  P.all_greedy = greedy ? 1 : 0;
  P.c = greedy ? 0.0f : (float)(1.4426950408889634074 / (double)temperature);
  P.chunks = 1;
  P.nvec = L.nvec;
  P.dchunks = L.dchunks;
  P.ntiles = L.ntiles;
  P.spin_limit = 1 << 16;
  P.out_tokens = out_tokens;
  P.num_accepted = num_accepted;
  P.slots = reinterpret_cast<unsigned long long*>(ws + L.off_slots);
  P.tiles = reinterpret_cast<float*>(ws + L.off_tiles);
  P.draw_done = reinterpret_cast<int*>(ws + L.off_draw_done);
  P.seq_flags = reinterpret_cast<int*>(ws + L.off_seq_flags);
  P.tok_logits = reinterpret_cast<float*>(ws + L.off_tok);
  unsigned long long* part = reinterpret_cast<unsigned long long*>(ws + L.off_part);

  auto grid_of = [&](int M, int NT) {
    const int MT = (M + kStBM - 1) / kStBM;
    const long long per_xcd = (NT + kXcds - 1) / kXcds;  // vocabulary tiles per XCD
    return std::make_pair(MT, (unsigned)(per_xcd * MT * kXcds));
  };
  // stage events: before the statistics GEMMs, then after them, after the
  // merge, and after the draw
  int e = 0;
  auto stage = [&]() {
    if (stage_events != nullptr && e < n_stage_events)
      return hipEventRecord(stage_events[e++], stream) == hipSuccess;
    return true;
  };
  if (!stage()) return SV_EHIP;
  // statistics of the draft rows and of the target rows, one launch
  LmPair S{};
  unsigned blocks_stats = 0;
  {
    LmGemm G{};
    G.V = V;
    G.NT = L.NT;
    G.part = part;
    G.tok_logits = P.tok_logits;
    G.K = K;
    G.tokens = draft_tokens;
    G.c = P.c;
    if (total_draft > 0 && !greedy) {
      auto [MT, blocks] = grid_of(total_draft, L.NT);
      G.H = static_cast<const uint16_t*>(hidden_draft);
      G.W = static_cast<const uint16_t*>(weight_draft);
      G.D = d_draft;
      G.M = total_draft;
      G.MT = MT;
      G.unit0 = 0;
      G.target = 0;
      G.out = ldraft;
      S.g[0] = G;
      S.n0 = (int)blocks;
      blocks_stats = blocks;
    }
    auto [MT, blocks] = grid_of(rows, L.NT);
    G.H = static_cast<const uint16_t*>(hidden_target);
    G.W = static_cast<const uint16_t*>(weight_target);
    G.D = d_target;
    G.M = rows;
    G.MT = MT;
    G.unit0 = total_draft;
    G.target = 1;
    // greedy: the draw reads no rows, so only the diag caller's are stored
    G.out = greedy ? logits_target : ltarget;
    if (blocks_stats == 0) {  // the target rows alone
      S.g[0] = G;
      S.n0 = (int)blocks;
    } else {
      S.g[1] = G;
    }
    blocks_stats += blocks;
  }
  if (greedy)
    hipLaunchKernelGGL(k_lm_stats<true>, dim3(blocks_stats), dim3(kStThreads), 0, stream, S);
  else
    hipLaunchKernelGGL(k_lm_stats<false>, dim3(blocks_stats), dim3(kStThreads), 0, stream, S);
  if (hipGetLastError() != hipSuccess || !stage()) return SV_EHIP;
  if (greedy) {
    // the target rows' argmax partials; the decision and the outputs are the
    // draw kernel's
    hipLaunchKernelGGL(k_lm_merge_am, dim3((unsigned)rows), dim3(kThreads), 0, stream, part,
                       P.slots, L.NT, (long long)total_draft);
  } else {
    hipLaunchKernelGGL(k_lm_merge, dim3((unsigned)(total_draft + rows)), dim3(kThreads), 0,
                       stream, part, P.slots, L.NT, P.c);
  }
  if (hipGetLastError() != hipSuccess || !stage()) return SV_EHIP;
  Plan DL{};
  DL.draw_blocks = (long long)B * L.dchunks;
  if (launch_draw_f32(L.nvec != V, P, DL, stream) != hipSuccess) return SV_EHIP;
  while (e < n_stage_events && stage_events != nullptr)
    if (!stage()) return SV_EHIP;
  return SV_OK;
}

}  // namespace

extern "C" int spec_verify_lmhead(const void* hidden_draft, const void* weight_draft, int d_draft,
                                  const void* hidden_target, const void* weight_target,
                                  int d_target, const int32_t* draft_tokens,
                                  const float* uniforms, int B, int K, int V, float temperature,
                                  int32_t* out_tokens, int32_t* num_accepted, void* workspace,
                                  size_t workspace_bytes, hipStream_t stream,
                                  hipEvent_t* stage_events, int n_stage_events) {
  return run_lmhead(hidden_draft, weight_draft, d_draft, hidden_target, weight_target, d_target,
                    draft_tokens, uniforms, B, K, V, temperature, out_tokens, num_accepted,
                    workspace, workspace_bytes, stream, stage_events, n_stage_events, nullptr,
                    nullptr);
}

extern "C" int spec_verify_lmhead_diag(const void* hidden_draft, const void* weight_draft,
                                       int d_draft, const void* hidden_target,
                                       const void* weight_target, int d_target,
                                       const int32_t* draft_tokens, const float* uniforms, int B,
                                       int K, int V, float temperature, int32_t* out_tokens,
                                       int32_t* num_accepted, void* workspace,
                                       size_t workspace_bytes, hipStream_t stream,
                                       hipEvent_t* stage_events, int n_stage_events,
                                       const sv_lmhead_diag* diag) {
  return run_lmhead(hidden_draft, weight_draft, d_draft, hidden_target, weight_target, d_target,
                    draft_tokens, uniforms, B, K, V, temperature, out_tokens, num_accepted,
                    workspace, workspace_bytes, stream, stage_events, n_stage_events,
                    diag != nullptr ? diag->logits_draft : nullptr,
                    diag != nullptr ? diag->logits_target : nullptr);
}
