// Internal interface between the C ABI (sv_api.cpp) and the kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "spec_verify.h"

namespace sv {

enum { kJobNone = 0, kJobResidual = 1, kJobBonus = 2 };

// Final draw of one sequence, written by k_decide, read by the draw kernels.
struct alignas(16) Job {
  int mode;     // kJob*
  int n;        // accepted drafts
  int qrow;     // draft row of position n (residual only)
  int prow;     // target row of position n
  int out_idx;  // output slot of the drawn token
  float Rq, invSq, Rp, invSp;  // references R = fp32(max*c) and 1/S of both rows
  float u;      // the resample-or-bonus uniform
  int pad[6];
};
static_assert(sizeof(Job) == 64, "Job is one 64-byte record");

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
  int B, K, V, total_draft;
  int all_greedy;
  float c;                 // log2(e) / temperature (0 if all greedy)
  int chunks;              // V-chunks per row in k_row_stats
  int chunk_vecs;          // vectors (or elements) per chunk
  int nvec;                // vectors (or elements) per row
  int ntiles;              // draw tiles per row (kTileElems elements each)
  int tile_chunks;         // k_resid_tiles blocks per sequence
  int tiles_per_chunk;
  int32_t* out_tokens;
  int32_t* num_accepted;
  float4* partials;        // [target rows * chunks]
  Job* jobs;               // [B]
  float* tile_sums;        // [B * ntiles]
  DiagPtrs diag;
};

// Grid sizes and workspace offsets of one call.
struct Plan {
  int chunks;
  int ntiles;
  int tiles_per_chunk;
  int tile_chunks;
  long long stats_blocks;
  long long tile_blocks;
  bool any_sampling;
  size_t off_jobs, off_partials, off_tiles, total_bytes;
};

hipError_t launch(int dtype, bool vec, const Params& P, const Plan& L, hipStream_t s,
                  hipEvent_t* ev, int nev);
hipError_t fill_zero(void* p, size_t bytes, hipStream_t s);

}  // namespace sv
