// Internal interface between the C ABI (sv_api.hip) and the kernel (sv_verify.hip).
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "spec_verify.h"

namespace sv {

constexpr int kThreads = 256;             // threads per block (4 waves)
constexpr int kBatch = 4;                 // 16-byte vectors per thread in flight per batch
constexpr int kTileVecs = kThreads;       // draw tile = one vector per thread
constexpr int kChunkVecs = 16 * kTileVecs;  // vectors of one row per stats block (64 KB)
constexpr int kDrawVecs = kBatch * kTileVecs;  // vectors of each row per draw block
constexpr int kTilesPerDraw = kDrawVecs / kTileVecs;
constexpr int kDecideLag = 16;            // draw chunk 0 of sequence b (which decides)
                                          // follows the stats of sequence b + kDecideLag
constexpr int kDrawLag = 20;              // its other draw chunks follow the stats of
                                          // sequence b + kDrawLag

// Per-sequence status bits raised by any block (cleared when the sequence ends).
enum { kSeqFlagTimeout = 1 };

enum { kJobNone = 0, kJobResidual = 1, kJobBonus = 2 };

// Final draw of one sequence, published by its deciding block.
struct alignas(16) Job {
  int mode;      // kJobNone / kJobResidual / kJobBonus
  int n;         // accepted drafts = position of the draw
  int prow;      // target row of position n
  int qrow;      // draft row of position n (residual only)
  float Rq, invSq, Rp, invSp;  // references R = fp32(max*c) and 1/S of both rows
  float u;       // the resample-or-bonus uniform
  int out_idx;   // output slot of the drawn token
  int pad[6];
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
  int dchunks;             // draw blocks per sequence
  int nvec;                // vectors (or elements, scalar path) per row
  int ntiles;              // draw tiles per row = dchunks * kTilesPerDraw
  int lag0, lag1;          // draw chunk 0 / other chunks of sequence b follow the
                           // stats blocks of sequence b + lag0 / b + lag1
  int spin_limit;          // bound of every wait (iterations)
  int32_t* out_tokens;
  int32_t* num_accepted;
  // Chunk partial of (target row, draft|target, chunk), 64-bit, 0 = not yet
  // published: sampling (max, sum) floats; greedy (max, tagged argmax).
  unsigned long long* slots;  // [rows * 2 * chunks]
  float* tiles;            // [B * ntiles] draw-weight tile sums
  Job* jobs;               // [B]
  int* job_ready;          // [B]
  int* draw_done;          // [B] draw blocks finished per sequence
  int* seq_flags;          // [B]
  DiagPtrs diag;
};

// Grid size and workspace offsets of one call.
struct Plan {
  int chunks, dchunks;
  long long blocks;
  size_t off_slots, off_tiles, off_jobs, off_job_ready, off_draw_done, off_seq_flags,
      total_bytes;
};

hipError_t launch(int dtype, bool vec, const Params& P, const Plan& L, hipStream_t s,
                  hipEvent_t* ev, int nev);
hipError_t fill_zero(void* p, size_t bytes, hipStream_t s);

}  // namespace sv
