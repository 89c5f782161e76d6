// C ABI of the verification library: argument checks, workspace layout and the
// launch of the kernels (sv_fused.hip without filters, sv_verify.hip with
// filters or for rows longer than the one-kernel step takes). Nothing here touches the device
// before every argument has been checked.
#include <limits.h>
#include <math.h>
#include <stdint.h>

#include <algorithm>
#include <atomic>
#include <cstdint>
#include <mutex>

#include "spec_verify.h"
#include "sv_launch.h"

namespace {

constexpr size_t kAlign = 256;
constexpr int kMaxV = 1 << 30;             // a greedy partial holds a 30-bit argmax
constexpr int kDefaultSpinLimit = 1 << 16;  // iterations of a bounded wait (~1 us each)

size_t align_up(size_t x) { return (x + kAlign - 1) / kAlign * kAlign; }

int esize_of(int dtype) { return dtype == SV_F32 ? 4 : 2; }

// Vectors per stats block for rows of nvec vectors: min_steps batches, grown
// so that no row has more than kMaxChunks chunks.
long long chunk_vecs_for(long long nvec, int min_steps) {
  const long long per = (long long)sv::kStepVecs * sv::kMaxChunks;
  long long steps = (nvec + per - 1) / per;
  if (steps < min_steps) steps = min_steps;
  return steps * sv::kStepVecs;
}

bool topk_active(int V, int top_k) { return top_k > 0 && top_k < V; }

bool filters_active(int V, int top_k, float top_p) {
  return topk_active(V, top_k) || top_p < 1.0f;
}

// (value, id) pairs per chunk record of a filtered row: k plus room for ties.
int kcap_for(int top_k) { return (top_k + 256 + 63) / 64 * 64; }

// Workspace layout (per call):
//   draw_done[B], seq_flags[B]             per-sequence counter and status bits
//   slots[(total_draft + rows) * cmax]     64-bit chunk partials (greedy rows, and
//                                          every row when no filter is active);
//                                          zero means "not yet published"
//   tiles[B * dmax * tiles per draw block] draw-weight tile sums (separate kernels)
//   draws[B * 2 * dmax]                    slice weight sums of the final draw
//                                          (one-kernel step)
//   beta_part[total_draft * cmax]          chunk sums of min(p, q) (acceptance
//   beta_cnt[total_draft]                  statistics) and per-pair counters
// and with top-k active:
//   rec[(total_draft + rows) * cmax * rec_words]  chunk records of sampling rows
//   rowres[total_draft + rows]                    kept-set statistics per row
//   kept[rows * kKeptWords]                       kept set of each target row
// Every region must be zero when a call starts (counters, flags, partials,
// tile and weight sums, and with filters the records, row results and kept
// lists); the blocks that read them return them to zero, so the layout may
// differ from call to call. The regions are sized for the scalar path (one
// element per vector), which has the most chunks: a row of nvec <= V vectors
// never has more than cmax chunks.
bool make_plan(int B, int total_draft, int V, int top_k, float top_p, size_t ws_bytes,
               sv::Plan& L) {
  if (B < 0 || total_draft < 0 || V < 1 || V > kMaxV) return false;
  const long long rows = (long long)total_draft + B;
  if (rows > INT_MAX) return false;
  const size_t units = (size_t)(total_draft + rows);
  const bool filt = topk_active(V, top_k) && top_k <= SV_MAX_TOP_K;
  const bool row_results = filt || top_p < 1.0f;
  long long cmax;
  if (filt) {
    cmax = ((long long)V + sv::kFiltChunkVecs - 1) / sv::kFiltChunkVecs;
  } else {
    // the smallest statistics chunk any call takes is one batch
    cmax = ((long long)V + sv::kStepVecs - 1) / sv::kStepVecs;
    if (cmax > sv::kMaxChunks) cmax = sv::kMaxChunks;
  }
  L.cmax = cmax;
  const long long dmax = ((long long)V + sv::kDrawVecs - 1) / sv::kDrawVecs;
  size_t off = 0;
  L.off_draw_done = off;
  off += align_up((size_t)B * 4);
  L.off_seq_flags = off;
  off += align_up((size_t)B * 4);
  L.off_slots = off;
  off += align_up(units * (size_t)cmax * 8);
  L.off_tiles = off;
  off += align_up((size_t)B * (size_t)dmax * sv::kTilesPerDraw * 4);
  L.off_draws = off;
  off += align_up((size_t)B * 2 * (size_t)dmax * 8);
  L.off_beta_part = off;
  off += align_up((size_t)total_draft * (size_t)cmax * 4);
  L.off_beta_cnt = off;
  off += align_up((size_t)total_draft * 4);
  L.off_rec = L.off_rowres = L.off_kept = off;
  if (filt) {
    const size_t rec_words = sv::kRecHeader + 2 * (size_t)kcap_for(top_k);
    off += align_up(units * (size_t)cmax * rec_words * 4);
    L.off_kept = off;
    off += align_up((size_t)rows * sv::kKeptWords * 4);
  }
  if (row_results) {
    L.off_rowres = off;
    off += align_up(units * sizeof(sv::RowRes));
  }
  L.total_bytes = off;
  return off <= ws_bytes;
}

size_t required_bytes(int B, int total_draft, int V, int top_k, float top_p) {
  sv::Plan L;
  if (!make_plan(B, total_draft, V, top_k, top_p, SIZE_MAX, L)) return 0;
  return L.total_bytes > 0 ? L.total_bytes : kAlign;
}


bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }

// Blocks of the one-kernel step one device holds at once (compute units times
// the kernel's occupancy), per device and kernel instance (3 dtypes x vector
// or scalar path). Facts about the device, looked up on first use and kept:
// no call's data is stored. 0 means not known yet; a racing first lookup
// stores the same value twice.
constexpr int kCapDevices = 64;
std::atomic<long long> fused_cap_cache[kCapDevices][6];

long long fused_capacity_of(hipStream_t stream, int dtype, bool vec) {
  int dev = 0;
  if (hipStreamGetDevice(stream, &dev) != hipSuccess) return 0;
  const int slot = dtype * 2 + (vec ? 1 : 0);
  if (dev < 0 || dev >= kCapDevices || slot < 0 || slot >= 6) return 0;
  long long cap = fused_cap_cache[dev][slot].load(std::memory_order_relaxed);
  if (cap > 0) return cap;
  int cus = 0;
  if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
      cus <= 0)
    return 0;
  cap = sv::fused_capacity(dtype, vec, cus);
  // keep the compute-unit count with it (capacity - cus is what the placement uses)
  if (cap > 0) fused_cap_cache[dev][slot].store(cap * 1024 + cus, std::memory_order_relaxed);
  return cap * 1024 + cus;
}

// Workspace of spec_verify_noalloc: one fixed array per device. In host code
// `scratch` names a host-side stand-in, never the device memory; the device
// address of each device's copy is looked up once, with that device current,
// and kept in scratch_ptr.
static __device__ __align__(256) unsigned char scratch[SV_NOALLOC_SCRATCH_BYTES];
constexpr int kMaxDevices = 64;
std::mutex scratch_mu;
void* scratch_ptr[kMaxDevices];

// Device address of `scratch` on the stream's device (SV_OK, or SV_EHIP /
// SV_EUNSUPPORTED if it cannot be found).
int scratch_of(hipStream_t stream, void** out) {
  int dev = 0;
  if (hipStreamGetDevice(stream, &dev) != hipSuccess) return SV_EHIP;
  if (dev < 0 || dev >= kMaxDevices) return SV_EUNSUPPORTED;
  std::lock_guard<std::mutex> lock(scratch_mu);
  if (scratch_ptr[dev] == nullptr) {
    int cur = 0;
    if (hipGetDevice(&cur) != hipSuccess) return SV_EHIP;
    if (cur != dev && hipSetDevice(dev) != hipSuccess) return SV_EHIP;
    void* p = nullptr;
    const hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (cur != dev && hipSetDevice(cur) != hipSuccess) return SV_EHIP;
    if (e != hipSuccess || p == nullptr) return SV_EHIP;
    scratch_ptr[dev] = p;
  }
  *out = scratch_ptr[dev];
  return SV_OK;
}

int run_accept(const void* draft, const void* target, const int32_t* cu, int B, int total_draft,
               int V, float temperature, int top_k, float top_p, int dtype, float* beta,
               float* expected, void* workspace, size_t workspace_bytes, hipStream_t stream);

int run(const void* draft, const void* target, const int32_t* tokens, const float* uniforms,
        const int32_t* cu, const uint8_t* greedy, int B, int K, int total_draft, int V,
        float temperature, int top_k, float top_p, int dtype, int32_t* out_tokens,
        int32_t* num_accepted, void* workspace, size_t workspace_bytes, hipStream_t stream,
        const sv_diag* diag, bool noalloc = false) {
  if (dtype != SV_F32 && dtype != SV_F16 && dtype != SV_BF16) return SV_EDTYPE;
  if (B < 0 || V < 1 || total_draft < 0) return SV_EINVAL;
  if (cu == nullptr && (K < 0 || K > SV_MAX_K)) return SV_EINVAL;
  if (!(temperature >= 0.0f) || isinf(temperature)) return SV_EINVAL;
  if (!(top_p > 0.0f && top_p <= 1.0f)) return SV_EINVAL;
  if (B == 0) return SV_OK;
  const bool all_greedy = temperature == 0.0f;
  if (target == nullptr || out_tokens == nullptr || num_accepted == nullptr) return SV_EINVAL;
  if (total_draft > 0 && tokens == nullptr) return SV_EINVAL;
  if (total_draft > 0 && !all_greedy && draft == nullptr) return SV_EINVAL;
  if (!all_greedy && uniforms == nullptr) return SV_EINVAL;
  // Filters act on sampling rows: top-k (then top-p) through candidate records,
  // top-p alone through a radix descent over each whole row.
  const bool filt = !all_greedy && filters_active(V, top_k, top_p);
  const bool topk = filt && topk_active(V, top_k);
  if (topk && top_k > SV_MAX_TOP_K) return SV_EUNSUPPORTED;
  sv::Plan L;
  if (!make_plan(B, total_draft, V, topk ? top_k : 0, filt ? top_p : 1.0f, SIZE_MAX, L))
    return SV_EUNSUPPORTED;
  if (noalloc) {
    // the library's fixed array, cleared where this call uses it (every
    // region of the layout must read zero when the kernels start)
    if (L.total_bytes > SV_NOALLOC_SCRATCH_BYTES) return SV_ESCRATCH;
    const int rc = scratch_of(stream, &workspace);
    if (rc != SV_OK) return rc;
    workspace_bytes = SV_NOALLOC_SCRATCH_BYTES;
    if (sv::fill_zero(workspace, L.total_bytes, stream) != hipSuccess) return SV_EHIP;
  }
  if (workspace == nullptr || ((uintptr_t)workspace % kAlign) != 0 ||
      !make_plan(B, total_draft, V, topk ? top_k : 0, filt ? top_p : 1.0f, workspace_bytes, L))
    return SV_EWORKSPACE;

  const int es = esize_of(dtype);
  const int n_per_vec = 16 / es;
  const bool vec = ((size_t)V * es) % 16 == 0 && aligned16(target) &&
                   (draft == nullptr || aligned16(draft));
  sv::Params P{};
  P.draft = draft;
  P.target = target;
  P.tokens = tokens;
  P.uniforms = uniforms;
  P.cu = cu;
  P.greedy = greedy;
  P.B = B;
  P.K = (cu == nullptr) ? K : 0;
  P.V = V;
  P.total_draft = total_draft;
  P.rows = total_draft + B;
  P.all_greedy = all_greedy ? 1 : 0;
  P.c = all_greedy ? 0.0f : (float)(1.4426950408889634074 / (double)temperature);
  P.nvec = vec ? V / n_per_vec : V;
  P.dchunks = (P.nvec + sv::kDrawVecs - 1) / sv::kDrawVecs;
  // unfiltered rows of at most kMaxDrawSlices slices run as one kernel (with
  // larger statistics chunks)
  L.fused = !filt && P.dchunks <= sv::kMaxDrawSlices;
  // acceptance statistics as side outputs (both pointers, or neither)
  const bool want_beta =
      diag != nullptr && (diag->beta != nullptr || diag->expected_accepted != nullptr);
  if (want_beta && (diag->expected_accepted == nullptr ||
                    (total_draft > 0 && diag->beta == nullptr)))
    return SV_EINVAL;
  if (want_beta && !L.fused && (all_greedy || greedy != nullptr)) return SV_EUNSUPPORTED;
  int steps = sv::kChunkSteps;
  if (L.fused) {
    // about kFusedBlocks statistics blocks over the call (small batches take
    // smaller chunks to fill the chip), at most kFusedChunkSteps batches each
    const long long rows_read = (all_greedy ? 0LL : (long long)total_draft) + P.rows;
    const long long want = rows_read * P.nvec / ((long long)sv::kFusedBlocks * sv::kStepVecs);
    steps = (int)std::max(1LL, std::min((long long)sv::kFusedChunkSteps, want));
  }
  P.chunk_vecs = topk ? sv::kFiltChunkVecs : (int)chunk_vecs_for(P.nvec, steps);
  P.chunks = (P.nvec + P.chunk_vecs - 1) / P.chunk_vecs;
  if (P.chunks > L.cmax) return SV_EUNSUPPORTED;  // the workspace holds cmax chunks per row
  P.ntiles = P.dchunks * sv::kTilesPerDraw;
  // greedy-only calls skip the draft rows
  P.stats_block0 = all_greedy ? (long long)total_draft * P.chunks : 0;
  P.filt = filt ? 1 : 0;
  P.nucleus = (filt && !topk) ? 1 : 0;
  P.top_k = top_k;
  P.top_p = top_p;
  P.kcap = topk ? kcap_for(top_k) : 0;
  P.rec_words = sv::kRecHeader + 2 * P.kcap;
  P.out_tokens = out_tokens;
  P.num_accepted = num_accepted;
  char* ws = static_cast<char*>(workspace);
  P.rec = topk ? reinterpret_cast<unsigned*>(ws + L.off_rec) : nullptr;
  P.rowres = filt ? reinterpret_cast<sv::RowRes*>(ws + L.off_rowres) : nullptr;
  P.kept = topk ? reinterpret_cast<unsigned*>(ws + L.off_kept) : nullptr;
  P.slots = reinterpret_cast<unsigned long long*>(ws + L.off_slots);
  P.tiles = reinterpret_cast<float*>(ws + L.off_tiles);
  P.draws = reinterpret_cast<unsigned long long*>(ws + L.off_draws);
  P.draw_done = reinterpret_cast<int*>(ws + L.off_draw_done);
  P.seq_flags = reinterpret_cast<int*>(ws + L.off_seq_flags);
  P.spin_limit = (diag != nullptr && diag->spin_limit > 0) ? diag->spin_limit : kDefaultSpinLimit;
  P.full_wait = (diag != nullptr &&
                 (diag->row_max_draft || diag->row_logsum_draft || diag->row_max_target ||
                  diag->row_logsum_target || diag->ratio))
                    ? 1
                    : 0;
  L.chunks = P.chunks;
  L.chunk_vecs = P.chunk_vecs;
  L.dchunks = P.dchunks;
  L.stats_blocks = ((long long)total_draft + P.rows) * P.chunks - P.stats_block0;
  L.filter_blocks = filt ? (long long)total_draft + P.rows : 0;
  L.draw_blocks = (long long)B * P.dchunks;
  P.stats_blocks = L.stats_blocks;
  if ((long long)B + L.stats_blocks + L.draw_blocks > (long long)UINT32_MAX / sv::kThreads)
    return SV_EUNSUPPORTED;
  // Placement of the one-kernel step's draw blocks (see sv_fused.hip): ahead
  // of the last two positions' statistics of a dense batch when the chip holds
  // all of them at once with at least one block per compute unit to spare,
  // after all the statistics otherwise.
  P.draw_at = L.stats_blocks;
  if (L.fused && cu == nullptr && K >= 2) {
    const long long packed = fused_capacity_of(stream, dtype, vec);
    const long long cap = packed / 1024, cus = packed % 1024;
    if (cap > 0 && L.draw_blocks <= cap - cus) {
      const long long per_pos = (all_greedy ? 1LL : 2LL) * B * P.chunks;
      P.draw_at = (long long)(K - 1) * per_pos;
    }
  }
  hipEvent_t* ev = nullptr;
  int nev = 0;
  if (diag != nullptr) {
    P.diag.row_max_draft = diag->row_max_draft;
    P.diag.row_logsum_draft = diag->row_logsum_draft;
    P.diag.row_max_target = diag->row_max_target;
    P.diag.row_logsum_target = diag->row_logsum_target;
    P.diag.ratio = diag->ratio;
    P.diag.resid_Z = diag->resid_Z;
    ev = diag->stage_events;
    nev = diag->n_stage_events;
  }
  hipError_t err;
  if (L.fused) {
    P.keep_pair_partials = want_beta ? 1 : 0;
    // stage events: before the kernel, then (every further one) after it, or
    // with the acceptance statistics the second after the verification and
    // every further one after the statistics
    if (ev != nullptr && nev > 0 && hipEventRecord(ev[0], stream) != hipSuccess) return SV_EHIP;
    err = sv::launch_fused(dtype, vec, P, L, stream);
    if (err != hipSuccess) return SV_EHIP;
    if (want_beta) {
      if (ev != nullptr && nev > 1 && hipEventRecord(ev[1], stream) != hipSuccess) return SV_EHIP;
      // the second pass: min(p, q) over every pair, from the partials the
      // verification left (same chunking), then beta and E[n]
      P.beta = diag->beta;
      P.expected = diag->expected_accepted;
      P.beta_part = reinterpret_cast<float*>(ws + L.off_beta_part);
      P.beta_cnt = reinterpret_cast<int*>(ws + L.off_beta_cnt);
      P.filt = 0;
      if (sv::launch_accept(dtype, vec, P, L, stream) != hipSuccess) return SV_EHIP;
    }
    for (int e = want_beta ? 2 : 1; ev != nullptr && e < nev; ++e)
      if (hipEventRecord(ev[e], stream) != hipSuccess) return SV_EHIP;
    return SV_OK;
  }
  err = sv::launch(dtype, vec, P, L, stream, ev, want_beta ? std::min(nev, 4) : nev);
  if (err != hipSuccess) return SV_EHIP;
  if (want_beta) {
    // the acceptance statistics as their own passes (the verification has
    // returned the workspace to zero)
    const int rc = run_accept(draft, target, cu, B, total_draft, V, temperature, top_k, top_p,
                              dtype, diag->beta, diag->expected_accepted, workspace,
                              workspace_bytes, stream);
    if (rc != SV_OK) return rc;
    for (int e = 4; ev != nullptr && e < nev; ++e)
      if (hipEventRecord(ev[e], stream) != hipSuccess) return SV_EHIP;
  }
  return SV_OK;
}

int run_accept(const void* draft, const void* target, const int32_t* cu, int B, int total_draft,
               int V, float temperature, int top_k, float top_p, int dtype, float* beta,
               float* expected, void* workspace, size_t workspace_bytes, hipStream_t stream) {
  if (dtype != SV_F32 && dtype != SV_F16 && dtype != SV_BF16) return SV_EDTYPE;
  if (B < 0 || V < 1 || total_draft < 0) return SV_EINVAL;
  if (!(temperature > 0.0f) || isinf(temperature)) return SV_EINVAL;
  if (!(top_p > 0.0f && top_p <= 1.0f)) return SV_EINVAL;
  if (B == 0) return SV_OK;
  int K = 0;
  if (cu == nullptr) {
    if (total_draft % B != 0 || total_draft / B > SV_MAX_K) return SV_EINVAL;
    K = total_draft / B;
  }
  if (target == nullptr || expected == nullptr) return SV_EINVAL;
  if (total_draft > 0 && (draft == nullptr || beta == nullptr)) return SV_EINVAL;
  const bool filt = filters_active(V, top_k, top_p);
  const bool topk = filt && topk_active(V, top_k);
  if (topk && top_k > SV_MAX_TOP_K) return SV_EUNSUPPORTED;
  sv::Plan L;
  if (!make_plan(B, total_draft, V, topk ? top_k : 0, top_p, SIZE_MAX, L))
    return SV_EUNSUPPORTED;
  if (workspace == nullptr || ((uintptr_t)workspace % kAlign) != 0 ||
      !make_plan(B, total_draft, V, topk ? top_k : 0, top_p, workspace_bytes, L))
    return SV_EWORKSPACE;
  const int es = esize_of(dtype);
  const bool vec = ((size_t)V * es) % 16 == 0 && aligned16(target) &&
                   (draft == nullptr || aligned16(draft));
  sv::Params P{};
  P.draft = draft;
  P.target = target;
  P.cu = cu;
  P.B = B;
  P.K = K;
  P.V = V;
  P.total_draft = total_draft;
  P.rows = total_draft + B;
  P.c = (float)(1.4426950408889634074 / (double)temperature);
  P.nvec = vec ? V / (16 / es) : V;
  P.chunk_vecs = topk ? sv::kFiltChunkVecs : (int)chunk_vecs_for(P.nvec, sv::kChunkSteps);
  P.chunks = (P.nvec + P.chunk_vecs - 1) / P.chunk_vecs;
  if (P.chunks > L.cmax) return SV_EUNSUPPORTED;  // the workspace holds cmax chunks per row
  P.filt = filt ? 1 : 0;
  P.nucleus = (filt && !topk) ? 1 : 0;
  P.top_k = top_k;
  P.top_p = top_p;
  P.kcap = topk ? kcap_for(top_k) : 0;
  P.rec_words = sv::kRecHeader + 2 * P.kcap;
  char* ws = static_cast<char*>(workspace);
  P.rec = topk ? reinterpret_cast<unsigned*>(ws + L.off_rec) : nullptr;
  P.rowres = filt ? reinterpret_cast<sv::RowRes*>(ws + L.off_rowres) : nullptr;
  P.slots = reinterpret_cast<unsigned long long*>(ws + L.off_slots);
  P.skip_bonus = 1;
  P.beta = beta;
  P.expected = expected;
  P.beta_part = reinterpret_cast<float*>(ws + L.off_beta_part);
  P.beta_cnt = reinterpret_cast<int*>(ws + L.off_beta_cnt);
  P.draw_done = reinterpret_cast<int*>(ws + L.off_draw_done);  // pairs finished per sequence
  L.chunks = P.chunks;
  L.chunk_vecs = P.chunk_vecs;
  L.stats_blocks = ((long long)total_draft + P.rows) * P.chunks;
  L.filter_blocks = filt ? (long long)total_draft + P.rows : 0;
  P.stats_blocks = L.stats_blocks;
  if (L.stats_blocks > (long long)UINT32_MAX / sv::kThreads) return SV_EUNSUPPORTED;
  if (sv::launch_row_stats(dtype, vec, P, L, stream) != hipSuccess) return SV_EHIP;
  return sv::launch_accept(dtype, vec, P, L, stream) == hipSuccess ? SV_OK : SV_EHIP;
}

// Tile totals a sequence's draw may publish (tiles of 1024 vectors, the
// walk's block width; a row has at most min(V, kMultiMaxVecs) vectors), and
// the bytes of the walk's cross-block state after the statistics layout: a
// sync record and the tile totals per sequence.
int multi_tiles(int V) {
  const int vecs = V < sv::kMultiMaxVecs ? V : sv::kMultiMaxVecs;
  return (vecs + 1023) / 1024;
}
size_t multi_state_bytes(int B, int V) {
  return align_up((size_t)B * sv::kMultiSyncWords * 4) + align_up((size_t)B * multi_tiles(V) * 4);
}

bool multi_sizes(int B, int M, int K, int V, long long& seqs, long long& drafts) {
  if (B < 0 || M < 1 || M > SV_MAX_CHAINS || K < 0 || K > SV_MAX_K || V < 1) return false;
  seqs = (long long)B * M;
  drafts = seqs * K;
  return seqs * (K + 1) <= INT_MAX;
}

int run_multi(const void* draft, const void* target, const int32_t* tokens, const float* uniforms,
              int B, int M, int K, int V, float temperature, int top_k, float top_p, int dtype,
              int32_t* out_tokens, int32_t* num_accepted, int32_t* out_chain, void* workspace,
              size_t workspace_bytes, hipStream_t stream) {
  if (dtype != SV_F32 && dtype != SV_F16 && dtype != SV_BF16) return SV_EDTYPE;
  long long seqs, drafts;
  if (!multi_sizes(B, M, K, V, seqs, drafts)) return SV_EINVAL;
  if (!(temperature >= 0.0f) || isinf(temperature)) return SV_EINVAL;
  if (!(top_p > 0.0f && top_p <= 1.0f)) return SV_EINVAL;
  if (B == 0) return SV_OK;
  const bool all_greedy = temperature == 0.0f;
  if (target == nullptr || out_tokens == nullptr || num_accepted == nullptr) return SV_EINVAL;
  if (!all_greedy && uniforms == nullptr) return SV_EINVAL;
  if (K > 0 && (tokens == nullptr || (!all_greedy && draft == nullptr))) return SV_EINVAL;
  // filters as for one chain: top-k (then top-p) through candidate records and
  // the per-row cut, top-p alone through the nucleus pass
  const bool filt = !all_greedy && filters_active(V, top_k, top_p);
  const bool topk = filt && topk_active(V, top_k);
  if (topk && top_k > SV_MAX_TOP_K) return SV_EUNSUPPORTED;
  const int pk = topk ? top_k : 0;
  const float pp = filt ? top_p : 1.0f;
  sv::Plan L;
  if (!make_plan((int)seqs, (int)drafts, V, pk, pp, SIZE_MAX, L)) return SV_EUNSUPPORTED;
  if (workspace == nullptr || ((uintptr_t)workspace % kAlign) != 0 ||
      L.total_bytes + multi_state_bytes(B, V) > workspace_bytes)
    return SV_EWORKSPACE;
  const int es = esize_of(dtype);
  const bool vec = ((size_t)V * es) % 16 == 0 && aligned16(target) &&
                   (draft == nullptr || aligned16(draft));
  sv::Params P{};
  P.draft = draft;
  P.target = target;
  P.tokens = tokens;
  P.uniforms = uniforms;
  P.B = (int)seqs;
  P.K = K;
  P.V = V;
  P.total_draft = (int)drafts;
  P.rows = (int)(seqs * (K + 1));
  P.all_greedy = all_greedy ? 1 : 0;
  P.c = all_greedy ? 0.0f : (float)(1.4426950408889634074 / (double)temperature);
  P.nvec = vec ? V / (16 / es) : V;
  if (P.nvec > sv::kMultiMaxVecs) return SV_EUNSUPPORTED;  // the walk's tile sums
  P.chunk_vecs = topk ? sv::kFiltChunkVecs : (int)chunk_vecs_for(P.nvec, sv::kChunkSteps);
  P.chunks = (P.nvec + P.chunk_vecs - 1) / P.chunk_vecs;
  if (P.chunks > L.cmax) return SV_EUNSUPPORTED;
  P.stats_block0 = all_greedy ? (long long)P.total_draft * P.chunks : 0;  // no draft rows read
  P.filt = filt ? 1 : 0;
  P.nucleus = (filt && !topk) ? 1 : 0;
  P.top_k = top_k;
  P.top_p = top_p;
  P.kcap = topk ? kcap_for(top_k) : 0;
  P.rec_words = sv::kRecHeader + 2 * P.kcap;
  P.rec = topk ? reinterpret_cast<unsigned*>(reinterpret_cast<char*>(workspace) + L.off_rec)
               : nullptr;
  P.rowres = filt ? reinterpret_cast<sv::RowRes*>(reinterpret_cast<char*>(workspace) +
                                                  L.off_rowres)
                  : nullptr;
  P.kept = nullptr;  // the walk lists no kept sets
  P.out_tokens = out_tokens;
  P.num_accepted = num_accepted;
  P.slots = reinterpret_cast<unsigned long long*>(reinterpret_cast<char*>(workspace) + L.off_slots);
  P.spin_limit = kDefaultSpinLimit;
  P.M = M;
  P.out_chain = out_chain;
  char* ms = reinterpret_cast<char*>(workspace) + L.total_bytes;
  P.msync = reinterpret_cast<int*>(ms);
  P.mtiles = reinterpret_cast<float*>(ms + align_up((size_t)B * sv::kMultiSyncWords * 4));
  P.mtiles_stride = multi_tiles(V);
  L.chunks = P.chunks;
  L.chunk_vecs = P.chunk_vecs;
  L.stats_blocks = ((long long)P.total_draft + P.rows) * P.chunks - P.stats_block0;
  L.filter_blocks = filt ? (long long)P.total_draft + P.rows : 0;
  P.stats_blocks = L.stats_blocks;
  if (L.stats_blocks > (long long)INT_MAX / sv::kThreads) return SV_EUNSUPPORTED;
  if (sv::launch_row_stats(dtype, vec, P, L, stream) != hipSuccess) return SV_EHIP;
  return sv::launch_multi(dtype, vec, P, stream) == hipSuccess ? SV_OK : SV_EHIP;
}

}  // namespace

extern "C" {

size_t spec_verify_multi_workspace_bytes(int B, int M, int K, int V, int top_k, float top_p) {
  long long seqs, drafts;
  if (!multi_sizes(B, M, K, V, seqs, drafts)) return 0;
  if (!(top_p > 0.0f && top_p <= 1.0f)) return 0;
  const bool topk = topk_active(V, top_k) && top_k <= SV_MAX_TOP_K;
  sv::Plan L;
  if (!make_plan((int)seqs, (int)drafts, V, topk ? top_k : 0, top_p, SIZE_MAX, L)) return 0;
  return L.total_bytes + multi_state_bytes(B, V);
}

int spec_verify_multi(const void* draft_logits, const void* target_logits,
                      const int32_t* draft_tokens, const float* uniforms, int B, int M, int K,
                      int V, float temperature, int top_k, float top_p, sv_dtype dtype,
                      int32_t* out_tokens, int32_t* num_accepted, int32_t* out_chain,
                      void* workspace, size_t workspace_bytes, hipStream_t stream) {
  return run_multi(draft_logits, target_logits, draft_tokens, uniforms, B, M, K, V, temperature,
                   top_k, top_p, (int)dtype, out_tokens, num_accepted, out_chain, workspace,
                   workspace_bytes, stream);
}

const char* spec_verify_strerror(int code) {
  switch (code) {
    case SV_OK: return "ok";
    case SV_EINVAL: return "invalid argument (null pointer, size, K, temperature or top_p)";
    case SV_EDTYPE: return "unknown dtype";
    case SV_EWORKSPACE: return "workspace null, not 256-byte aligned, or too small";
    case SV_EHIP: return "HIP launch or event record failed";
    case SV_EUNSUPPORTED: return "request outside this build's limits";
    case SV_ESCRATCH: return "call needs more than the fixed scratch array holds";
    default: return "unknown code";
  }
}

size_t spec_verify_workspace_bytes(int B, int total_draft_rows, int V, int top_k, float top_p) {
  (void)top_p;
  return required_bytes(B, total_draft_rows, V, top_k, top_p);
}

int spec_verify_workspace_init(void* workspace, size_t workspace_bytes, hipStream_t stream) {
  if (workspace_bytes == 0) return SV_OK;
  if (workspace == nullptr || ((uintptr_t)workspace % kAlign) != 0) return SV_EWORKSPACE;
  return sv::fill_zero(workspace, workspace_bytes, stream) == hipSuccess ? SV_OK : SV_EHIP;
}

int spec_verify_num_stages(int top_k, float top_p) {
  return (top_k > 0 || top_p < 1.0f) ? 3 : 1;
}

int spec_verify(const void* draft_logits, const void* target_logits, const int32_t* draft_tokens,
                const float* uniforms, int B, int K, int V, float temperature, int top_k,
                float top_p, sv_dtype dtype, int32_t* out_tokens, int32_t* num_accepted,
                void* workspace, size_t workspace_bytes, hipStream_t stream) {
  if (K < 0 || K > SV_MAX_K || B < 0) return SV_EINVAL;
  const long long total = (long long)B * K;
  if (total > INT_MAX) return SV_EINVAL;
  return run(draft_logits, target_logits, draft_tokens, uniforms, nullptr, nullptr, B, K,
             (int)total, V, temperature, top_k, top_p, (int)dtype, out_tokens, num_accepted,
             workspace, workspace_bytes, stream, nullptr);
}

int spec_verify_noalloc(const void* draft_logits, const void* target_logits,
                        const int32_t* draft_tokens, const float* uniforms, int B, int K, int V,
                        float temperature, int top_k, float top_p, sv_dtype dtype,
                        int32_t* out_tokens, int32_t* num_accepted, hipStream_t stream) {
  if (K < 0 || K > SV_MAX_K || B < 0) return SV_EINVAL;
  const long long total = (long long)B * K;
  if (total > INT_MAX) return SV_EINVAL;
  return run(draft_logits, target_logits, draft_tokens, uniforms, nullptr, nullptr, B, K,
             (int)total, V, temperature, top_k, top_p, (int)dtype, out_tokens, num_accepted,
             nullptr, 0, stream, nullptr, true);
}

int spec_verify_ragged(const void* draft_logits, const void* target_logits,
                       const int32_t* draft_tokens, const float* uniforms,
                       const int32_t* cu_draft, const uint8_t* greedy, int B,
                       int total_draft_rows, int V, float temperature, int top_k, float top_p,
                       sv_dtype dtype, int32_t* out_tokens, int32_t* num_accepted,
                       void* workspace, size_t workspace_bytes, hipStream_t stream) {
  if (cu_draft == nullptr) return SV_EINVAL;
  return run(draft_logits, target_logits, draft_tokens, uniforms, cu_draft, greedy, B, 0,
             total_draft_rows, V, temperature, top_k, top_p, (int)dtype, out_tokens,
             num_accepted, workspace, workspace_bytes, stream, nullptr);
}

int spec_verify_diag(const void* draft_logits, const void* target_logits,
                     const int32_t* draft_tokens, const float* uniforms, const int32_t* cu_draft,
                     const uint8_t* greedy, int B, int total_draft_rows, int V, float temperature,
                     int top_k, float top_p, sv_dtype dtype, int32_t* out_tokens,
                     int32_t* num_accepted, void* workspace, size_t workspace_bytes,
                     hipStream_t stream, const sv_diag* diag) {
  if (cu_draft == nullptr) return SV_EINVAL;
  return run(draft_logits, target_logits, draft_tokens, uniforms, cu_draft, greedy, B, 0,
             total_draft_rows, V, temperature, top_k, top_p, (int)dtype, out_tokens,
             num_accepted, workspace, workspace_bytes, stream, diag);
}

int spec_verify_accept_stats(const void* draft_logits, const void* target_logits,
                             const int32_t* cu_draft, int B, int total_draft_rows, int V,
                             float temperature, int top_k, float top_p, sv_dtype dtype,
                             float* beta, float* expected_accepted, void* workspace,
                             size_t workspace_bytes, hipStream_t stream) {
  return run_accept(draft_logits, target_logits, cu_draft, B, total_draft_rows, V, temperature,
                    top_k, top_p, (int)dtype, beta, expected_accepted, workspace,
                    workspace_bytes, stream);
}

}  // extern "C"
