// C ABI of the verification library: argument checks, workspace layout and the
// launch of the kernels in sv_kernels.hip. Nothing here touches the device
// before every argument has been checked.
#include <limits.h>
#include <math.h>
#include <stdint.h>

#include "spec_verify.h"
#include "sv_launch.h"

namespace {

constexpr size_t kAlign = 256;
constexpr int kStatsTargetBlocks = 2048;   // aim: several blocks per CU
constexpr int kMinChunkElems = 8192;       // smallest V-chunk worth a block
constexpr int kMaxChunks = 16;
constexpr int kTileElems = 2048;           // must match sv::kTileElems
constexpr int kTilesPerBlock = 4;          // one tile per wave of k_resid_tiles

size_t align_up(size_t x) { return (x + kAlign - 1) / kAlign * kAlign; }

int esize_of(int dtype) { return dtype == SV_F32 ? 4 : 2; }

bool make_plan(int B, int total_draft, int V, sv::Plan& L) {
  if (B < 0 || total_draft < 0 || V < 1) return false;
  const long long rows_t = (long long)total_draft + B;
  if (rows_t > INT_MAX) return false;
  long long chunks = 1;
  if (rows_t > 0) {
    const long long want = (kStatsTargetBlocks + rows_t - 1) / rows_t;
    long long cap = V / kMinChunkElems;
    if (cap < 1) cap = 1;
    if (cap > kMaxChunks) cap = kMaxChunks;
    chunks = want < cap ? want : cap;
    if (chunks < 1) chunks = 1;
  }
  L.chunks = (int)chunks;
  L.ntiles = (int)(((long long)V + kTileElems - 1) / kTileElems);
  L.tiles_per_chunk = kTilesPerBlock;
  L.tile_chunks = (L.ntiles + kTilesPerBlock - 1) / kTilesPerBlock;
  L.stats_blocks = rows_t * chunks;
  L.tile_blocks = (long long)B * L.tile_chunks;
  // grid x * block must stay below 2^32 threads
  if (L.stats_blocks * 256 > (long long)UINT32_MAX || L.tile_blocks * 256 > (long long)UINT32_MAX)
    return false;
  size_t off = 0;
  L.off_jobs = off;
  off = align_up(off + (size_t)B * sizeof(sv::Job));
  L.off_partials = off;
  off = align_up(off + (size_t)rows_t * (size_t)chunks * 16);
  L.off_tiles = off;
  off = align_up(off + (size_t)B * (size_t)L.ntiles * 4);
  L.total_bytes = off;
  return true;
}

bool filters_active(int V, int top_k, float top_p) {
  return (top_k > 0 && top_k < V) || top_p < 1.0f;
}

bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }

int run(const void* draft, const void* target, const int32_t* tokens, const float* uniforms,
        const int32_t* cu, const uint8_t* greedy, int B, int K, int total_draft, int V,
        float temperature, int top_k, float top_p, int dtype, int32_t* out_tokens,
        int32_t* num_accepted, void* workspace, size_t workspace_bytes, hipStream_t stream,
        const sv_diag* diag) {
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
  if (!all_greedy && filters_active(V, top_k, top_p)) {
    if (top_k > SV_MAX_TOP_K) return SV_EUNSUPPORTED;
    return SV_EUNSUPPORTED;  // top-k / top-p path not in this build yet
  }
  sv::Plan L;
  if (!make_plan(B, total_draft, V, L)) return SV_EINVAL;
  if (workspace == nullptr || ((uintptr_t)workspace % kAlign) != 0 ||
      workspace_bytes < L.total_bytes)
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
  P.all_greedy = all_greedy ? 1 : 0;
  P.c = all_greedy ? 0.0f : (float)(1.4426950408889634074 / (double)temperature);
  P.nvec = vec ? V / n_per_vec : V;
  P.chunks = L.chunks;
  P.chunk_vecs = (P.nvec + L.chunks - 1) / L.chunks;
  P.ntiles = L.ntiles;
  P.tile_chunks = L.tile_chunks;
  P.tiles_per_chunk = L.tiles_per_chunk;
  P.out_tokens = out_tokens;
  P.num_accepted = num_accepted;
  char* ws = static_cast<char*>(workspace);
  P.jobs = reinterpret_cast<sv::Job*>(ws + L.off_jobs);
  P.partials = reinterpret_cast<float4*>(ws + L.off_partials);
  P.tile_sums = reinterpret_cast<float*>(ws + L.off_tiles);
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
  L.any_sampling = !all_greedy;
  const hipError_t err = sv::launch(dtype, vec, P, L, stream, ev, nev);
  return err == hipSuccess ? SV_OK : SV_EHIP;
}

}  // namespace

extern "C" {

const char* spec_verify_strerror(int code) {
  switch (code) {
    case SV_OK: return "ok";
    case SV_EINVAL: return "invalid argument (null pointer, size, K, temperature or top_p)";
    case SV_EDTYPE: return "unknown dtype";
    case SV_EWORKSPACE: return "workspace null, not 256-byte aligned, or too small";
    case SV_EHIP: return "HIP launch or event record failed";
    case SV_EUNSUPPORTED: return "request outside this build's limits";
    default: return "unknown code";
  }
}

size_t spec_verify_workspace_bytes(int B, int total_draft_rows, int V, int top_k, float top_p) {
  (void)top_k;
  (void)top_p;
  sv::Plan L;
  if (!make_plan(B, total_draft_rows, V, L)) return 0;
  return L.total_bytes;
}

int spec_verify_workspace_init(void* workspace, size_t workspace_bytes, hipStream_t stream) {
  if (workspace_bytes == 0) return SV_OK;
  if (workspace == nullptr || ((uintptr_t)workspace % kAlign) != 0) return SV_EWORKSPACE;
  return sv::fill_zero(workspace, workspace_bytes, stream) == hipSuccess ? SV_OK : SV_EHIP;
}

int spec_verify_num_stages(int top_k, float top_p) {
  (void)top_k;
  (void)top_p;
  return 4;
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

}  // extern "C"
