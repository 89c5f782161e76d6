// Internal interface between the C ABI (sv_api.hip) and the kernels
// (sv_fused.hip, sv_verify.hip).
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "spec_verify.h"

namespace sv {

constexpr int kThreads = 256;             // threads per block (4 waves)
constexpr int kBatch = 4;                 // 16-byte vectors per thread in flight per batch
constexpr int kTileVecs = kThreads;       // draw tile = one vector per thread
constexpr int kMultiMaxVecs = 1 << 18;    // vectors a row of spec_verify_multi may have
constexpr int kMultiSplit = 4;            // blocks that share one sequence's walk
constexpr int kMultiSyncWords = 16;       // per-sequence words of the walk's cross-block state
constexpr int kStepVecs = kBatch * kThreads;  // vectors of a row one batch covers
constexpr int kDrawVecs = kStepVecs;      // vectors of each row per draw block
constexpr int kTilesPerDraw = kDrawVecs / kTileVecs;
constexpr int kChunkSteps = 4;            // batches per stats block (64 KB of bf16)
constexpr int kFusedChunkSteps = 8;       // at most this many in the one-kernel step (128 KB)
constexpr int kFusedBlocks = 2048;        // statistics blocks the one-kernel step aims for
constexpr int kMaxChunks = 64;            // stats chunks per row (larger rows take
                                          // larger chunks)
// Filtered rows (top-k): a stats block keeps its whole chunk in registers.
constexpr int kFiltVpt = 8;               // vectors per thread of a filtered chunk
constexpr int kFiltChunkVecs = kFiltVpt * kThreads;
constexpr int kRecHeader = 8;             // header words of a chunk record
constexpr int kBoundMaxK = kThreads;      // largest k bounded by the per-thread maxima
constexpr int kHitMax = 512;              // candidate vectors a stats block stages in LDS
constexpr int kFilterMaxLevels = 1024;    // LDS entries of the per-row level sort (levels
                                          // above the k-th largest, plus its tie class)
constexpr int kFilterLdsKeys = 2048;      // record entries a filter block stages in LDS
constexpr int kFilterLdsChunks = 64;      // record headers a filter block stages in LDS
constexpr int kExplicitMax = 2048;        // candidates a filtered draw gathers in LDS
constexpr int kKeptWords = 2 + 2 * kExplicitMax;  // words of a target row's kept list
constexpr int kMaxDrawSlices = kThreads;  // draw blocks per sequence of the one-kernel
                                          // step (longer rows take the separate kernels)

// Chunk record of a filtered row: header then `kcap` (value bits, id) pairs.
//   [0] entries written   [1] value of an implicit tie class   [2] its count
//   [3] flags: 1 NaN or +inf seen, 2 the tie class is implicit (count only)
enum { kRecFlagBad = 1, kRecFlagImplicitTies = 2 };

// Per-row result of the filter pass: kept-set maximum, kept-set sum of
// 2^(l*c - R) (R = fp32(max*c)), threshold theta (kept iff l >= theta), flags.
struct RowRes {
  float m, s, theta;
  int flags;
};

// Per-sequence status bits raised by any block (cleared when the sequence ends).
enum { kSeqFlagTimeout = 1 };

enum { kJobNone = 0, kJobResidual = 1, kJobBonus = 2 };

// Final draw of one sequence (every draw block of the sequence derives it).
struct Job {
  int mode;      // kJobNone / kJobResidual / kJobBonus
  int n;         // accepted drafts = position of the draw
  int prow;      // target row of position n
  int qrow;      // draft row of position n (residual only)
  float Rq, invSq, Rp, invSp;  // references R = fp32(max*c) and 1/S of both rows
  float thr_q, thr_p;  // kept-set thresholds of both rows (-inf: no filter)
  float u;       // the resample-or-bonus uniform
  int out_idx;   // output slot of the drawn token
};

// Device pointers of the optional side outputs.
struct DiagPtrs {
  float* row_max_draft;
  float* row_logsum_draft;
  float* row_max_target;
  float* row_logsum_target;
  float* ratio;
  float* resid_Z;
};

struct Params {
  const void* draft;
  const void* target;
  const int32_t* tokens;
  const float* uniforms;
  const int32_t* cu;       // null: dense layout with K drafts per sequence
  const uint8_t* greedy;   // null: no per-sequence greedy mask
  int B, K, V, total_draft, rows;  // rows = total target rows
  int all_greedy;
  float c;                 // log2(e) / temperature (0 if all greedy)
  int chunks;              // stats blocks per row
  int chunk_vecs;          // vectors per stats block (a multiple of kStepVecs)
  int dchunks;             // draw blocks (vocabulary slices) per sequence
  int nvec;                // vectors (or elements, scalar path) per row
  int ntiles;              // draw tiles per row = dchunks * kTilesPerDraw
  long long stats_block0;  // first stats unit block (skips draft rows when all greedy;
                           // draft-then-target order)
  long long stats_blocks;  // stats blocks launched
  int spin_limit;          // bound of every wait (iterations)
  int full_wait;           // 1: decisions read every row (side outputs requested)
  int keep_pair_partials;  // 1: the one-kernel step leaves the partials of every
                           // sampling sequence's draft rows and non-bonus target
                           // rows for the acceptance statistics pass that follows
  int filt;                // 1: filters active (rows carry kept-set results)
  int nucleus;             // 1: top-p without top-k (no candidate records)
  int top_k;
  float top_p;
  int kcap;                // (value, id) pairs per chunk record
  int rec_words;           // words per chunk record = kRecHeader + 2 * kcap
  unsigned* rec;           // [(total_draft + rows) * chunks * rec_words] (filtered)
  // Kept set of each filtered target row, written by the filter pass for the
  // final draw: [0] entries listed, [1] 1 if the set is not listed in full (a
  // count-only tie class, or more than kExplicitMax ids), then (value bits,
  // id) pairs. Zero between calls.
  unsigned* kept;          // [rows * kKeptWords] (filtered)
  RowRes* rowres;          // [total_draft + rows] (filtered)
  int32_t* out_tokens;
  int32_t* num_accepted;
  // Chunk partials, 64-bit and never zero once written (zero: not yet
  // published; the readers return them to zero): sampling (max, sum) floats;
  // greedy (max value, tagged argmax and bad flag). Draft rows first, then
  // target rows, chunks innermost.
  unsigned long long* slots;  // [(total_draft + rows) * chunks]
  float* tiles;            // [B * ntiles] draw-weight tile sums
  int* draw_done;          // [B] blocks finished per sequence (zero between calls)
  int* seq_flags;          // [B] kSeqFlag* bits (zero between calls)
  // One-kernel step: slice weight sums of each sequence's final draw, 64-bit
  // (tag bit 63, float bits below), two sets of `dchunks` per sequence (the
  // residual, then the target row if the residual mass rounds to zero).
  unsigned long long* draws;  // [B * 2 * dchunks]
  long long draw_at;       // one-kernel step: statistics blocks ahead of the draw blocks
  DiagPtrs diag;
  // Acceptance statistics (spec_verify_accept_stats)
  int skip_bonus;          // 1: the statistics pass skips each sequence's bonus row
  float* beta;             // [total_draft] output: pass probability per draft position
  float* expected;         // [B] output: expected accepted drafts per sequence
  float* beta_part;        // [total_draft * chunks] chunk sums of min(p, q)
  int* beta_cnt;           // [total_draft] chunks finished per row pair (zero between calls)
  // Verification from LM-head hidden states (sv_lmhead.hip): the logit of
  // each statistics unit at its token (draft units: their own token; target
  // units at position i < K_b: token x_i), written by the GEMM epilogue, read
  // by the decision instead of the logit rows (the final draw reads the fp32
  // rows the GEMM stored, given as the two logit arrays).
  float* tok_logits;       // [total_draft + rows] or null
  // Several draft chains per sequence (sv_multi.hip): B above counts the
  // chains as sequences of the statistics pass (B = sequences * M).
  int M;                   // chains per sequence
  int32_t* out_chain;      // [B / M] the lowest chain holding the emitted prefix, or null
  int* msync;              // [B / M * kMultiSyncWords] the walk's cross-block state
  float* mtiles;           // [B / M * mtiles_stride] tile totals of a sequence's draw
  int mtiles_stride;
};

// Grid size and workspace offsets of one call.
struct Plan {
  int chunks, chunk_vecs, dchunks;
  long long cmax;  // chunks per row the workspace holds partials and records for
  bool fused;  // one kernel (k_verify) instead of statistics, filter and draw kernels
  long long stats_blocks, filter_blocks, draw_blocks;
  size_t off_slots, off_tiles, off_draws, off_draw_done, off_seq_flags, off_rec, off_rowres,
      off_kept, off_beta_part, off_beta_cnt, total_bytes;
};

// The separate statistics / filter / draw kernels (sv_verify.hip).
hipError_t launch(int dtype, bool vec, const Params& P, const Plan& L, hipStream_t s,
                  hipEvent_t* ev, int nev);
// The one-kernel unfiltered step (sv_fused.hip), and the number of its blocks
// the chip holds at once with `cus` compute units (0 if unknown).
hipError_t launch_fused(int dtype, bool vec, const Params& P, const Plan& L, hipStream_t s);
long long fused_capacity(int dtype, bool vec, int cus);
// Row statistics alone (the statistics pass, and the filter pass with top-k):
// the first stage of the acceptance statistics (sv_verify.hip).
hipError_t launch_row_stats(int dtype, bool vec, const Params& P, const Plan& L, hipStream_t s);
// The acceptance statistics after the row statistics (sv_accept.hip).
hipError_t launch_accept(int dtype, bool vec, const Params& P, const Plan& L, hipStream_t s);
hipError_t fill_zero(void* p, size_t bytes, hipStream_t s);
// Several draft chains: the walk after the statistics pass (sv_multi.hip).
hipError_t launch_multi(int dtype, bool vec, const Params& P, hipStream_t s);
// LM-head path (sv_lmhead.hip drives these from sv_verify.hip): the decision
// that picks the draw's hidden rows, and the draw over fp32 logit rows.
hipError_t launch_draw_f32(bool vec, const Params& P, const Plan& L, hipStream_t s);

}  // namespace sv
