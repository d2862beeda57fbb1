// C ABI of the ReLU linear self-attention forward pass (include/sana_linattn.h):
// argument checks, the work split, workspace layout and kernel launches.
// Every check runs on the host before the first HIP call.

#include "sana_linattn.h"

#include <cmath>
#include <cstdint>
#include <cstdlib>
#include <cstring>
#include <algorithm>

#include "linattn_internal.h"

namespace sana {
namespace {

constexpr int64_t kTargetReduceBlocks = 1024;  // 4 blocks (16 waves) per CU on 256 CUs
constexpr int64_t kTargetApplyBlocks = 2048;
constexpr int64_t kMinReduceChunk = 256;       // tokens: 8 tiles per wave at 2 sub-streams
constexpr int64_t kMinApplyChunk = 256;
constexpr int64_t kMaxReduceChunks = 64;
constexpr int64_t kMaxApplyChunks = 1 << 20;
constexpr int64_t kFusedMaxN = 1024;           // AUTO picks the fused kernel up to this N
constexpr size_t kAlign = 256;

int64_t cdiv(int64_t a, int64_t b) { return (a + b - 1) / b; }
int64_t clamp64(int64_t x, int64_t lo, int64_t hi) { return x < lo ? lo : (x > hi ? hi : x); }
size_t align_up(size_t x) { return (x + kAlign - 1) / kAlign * kAlign; }

bool overlaps(const void* a, size_t na, const void* b, size_t nb) {
  if (!a || !b || na == 0 || nb == 0) return false;
  const uintptr_t x = reinterpret_cast<uintptr_t>(a), y = reinterpret_cast<uintptr_t>(b);
  return x < y + nb && y < x + na;
}

bool misaligned(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) != 0; }

// Shape checks shared by every entry point. *tensor_bytes = bytes of one
// [B][N][H][d] tensor.
sana_status_t check_shape(int64_t B, int64_t N, int64_t H, int64_t d, int dtype,
                          size_t* tensor_bytes) {
  if (B < 1 || N < 1 || H < 1 || d < 1) return SANA_ERR_INVALID_ARG;
  if (d != kHeadDim) return SANA_ERR_UNSUPPORTED;
  if (dtype != SANA_DTYPE_F32 && dtype != SANA_DTYPE_BF16) return SANA_ERR_UNSUPPORTED;
  const int64_t item = dtype == SANA_DTYPE_F32 ? 4 : 2;
  int64_t t = 0;
  if (__builtin_mul_overflow(B, N, &t) || __builtin_mul_overflow(t, H, &t) ||
      __builtin_mul_overflow(t, d, &t) || __builtin_mul_overflow(t, item, &t) ||
      t >= (int64_t(1) << 62))
    return SANA_ERR_INVALID_ARG;
  // state and workspace sizes stay far below this once B*H fits
  int64_t bh = 0;
  if (__builtin_mul_overflow(B, H, &bh) || bh > (int64_t(1) << 40)) return SANA_ERR_INVALID_ARG;
  if (tensor_bytes) *tensor_bytes = static_cast<size_t>(t);
  return SANA_OK;
}

sana_status_t check_eps(float eps) {
  if (!std::isfinite(eps) || eps < 0.0f) return SANA_ERR_INVALID_ARG;
  return SANA_OK;
}

}  // namespace

Plan make_plan(int64_t B, int64_t N, int64_t H) {
  Plan p{};
  p.B = B;
  p.N = N;
  p.H = H;
  p.pairs = cdiv(H, kHeadsPerBlock);
  p.units = B * p.pairs;
  // Split-N reduction: enough chunks to fill the chip, each at least
  // kMinReduceChunk tokens. Once N >= kMinReduceChunk * red_chunks_max the
  // count no longer depends on N, nor does the workspace.
  p.red_chunks_max = clamp64(cdiv(kTargetReduceBlocks, p.units), 1, kMaxReduceChunks);
  const int64_t want = clamp64(cdiv(N, kMinReduceChunk), 1, p.red_chunks_max);
  p.red_chunk = cdiv(cdiv(N, want), kTile) * kTile;
  p.red_chunks = cdiv(N, p.red_chunk);
  const int64_t awant = clamp64(std::min(cdiv(kTargetApplyBlocks, p.units), cdiv(N, kMinApplyChunk)),
                                1, kMaxApplyChunks);
  p.app_chunk = cdiv(cdiv(N, awant), kTile) * kTile;
  p.app_chunks = cdiv(N, p.app_chunk);
  const size_t bh = static_cast<size_t>(B * H);
  p.partial_bytes = align_up(static_cast<size_t>(p.red_chunks_max) * bh * kStateFloats * 4);
  p.state_bytes = align_up(bh * kStateFloats * 4);
  p.workspace_bytes = p.partial_bytes + p.state_bytes;
  return p;
}

namespace {

sana_status_t check_workspace(const Plan& p, const void* ws, size_t ws_bytes) {
  if (p.workspace_bytes == 0) return SANA_OK;
  if (!ws || ws_bytes < p.workspace_bytes) return SANA_ERR_WORKSPACE;
  if ((reinterpret_cast<uintptr_t>(ws) & (kAlign - 1)) != 0) return SANA_ERR_ALIGNMENT;
  return SANA_OK;
}

sana_status_t to_status(hipError_t e) { return e == hipSuccess ? SANA_OK : SANA_ERR_HIP; }

bool use_fused(const Plan& p, int variant) {
  if (variant == SANA_VARIANT_FUSED) return true;
  if (variant == SANA_VARIANT_SPLIT) return false;
  return p.N <= kFusedMaxN;
}

sana_status_t run_state(const Plan& p, int dtype, const void* k, const void* v, float* state,
                        void* ws, hipStream_t stream) {
  float* partials = static_cast<float*>(ws);
  hipError_t e = launch_reduce(p, dtype, k, v, partials, stream);
  if (e != hipSuccess) return SANA_ERR_HIP;
  return to_status(launch_combine(p, partials, state, stream));
}

}  // namespace
}  // namespace sana

using sana::Plan;

extern "C" {

sana_status_t sana_linattn_workspace_size(int64_t B, int64_t N, int64_t H, int64_t d, int dtype,
                                          size_t* bytes) {
  if (!bytes) return SANA_ERR_INVALID_ARG;
  *bytes = 0;
  const sana_status_t s = sana::check_shape(B, N, H, d, dtype, nullptr);
  if (s != SANA_OK) return s;
  *bytes = sana::make_plan(B, N, H).workspace_bytes;
  return SANA_OK;
}

sana_status_t sana_linattn_state_size(int64_t B, int64_t H, int64_t d, size_t* bytes) {
  if (!bytes) return SANA_ERR_INVALID_ARG;
  *bytes = 0;
  const sana_status_t s = sana::check_shape(B, 1, H, d, SANA_DTYPE_F32, nullptr);
  if (s != SANA_OK) return s;
  *bytes = static_cast<size_t>(B * H) * sana::kStateFloats * 4;
  return SANA_OK;
}

sana_status_t sana_linattn_fwd_variant(const void* q, const void* k, const void* v, void* out,
                                       int64_t B, int64_t N, int64_t H, int64_t d, float eps,
                                       int dtype, int variant, void* workspace,
                                       size_t workspace_bytes, hipStream_t stream) {
  size_t tb = 0;
  sana_status_t s = sana::check_shape(B, N, H, d, dtype, &tb);
  if (s != SANA_OK) return s;
  if (variant != SANA_VARIANT_AUTO && variant != SANA_VARIANT_SPLIT && variant != SANA_VARIANT_FUSED)
    return SANA_ERR_UNSUPPORTED;
  if (!q || !k || !v || !out) return SANA_ERR_INVALID_ARG;
  if ((s = sana::check_eps(eps)) != SANA_OK) return s;
  if (sana::misaligned(q) || sana::misaligned(k) || sana::misaligned(v) || sana::misaligned(out))
    return SANA_ERR_ALIGNMENT;
  if (sana::overlaps(out, tb, q, tb) || sana::overlaps(out, tb, k, tb) ||
      sana::overlaps(out, tb, v, tb))
    return SANA_ERR_INVALID_ARG;
  const Plan p = sana::make_plan(B, N, H);
  if ((s = sana::check_workspace(p, workspace, workspace_bytes)) != SANA_OK) return s;
  if (sana::overlaps(out, tb, workspace, p.workspace_bytes)) return SANA_ERR_INVALID_ARG;

  (void)hipGetLastError();  // clear an unrelated earlier error
  if (sana::use_fused(p, variant))
    return sana::to_status(sana::launch_fused(p, dtype, q, k, v, out, eps, stream));
  float* state = reinterpret_cast<float*>(static_cast<char*>(workspace) + p.partial_bytes);
  if ((s = sana::run_state(p, dtype, k, v, state, workspace, stream)) != SANA_OK) return s;
  return sana::to_status(sana::launch_apply(p, dtype, q, state, out, eps, stream));
}

sana_status_t sana_linattn_fwd_profiled(const void* q, const void* k, const void* v, void* out,
                                        int64_t B, int64_t N, int64_t H, int64_t d, float eps,
                                        int dtype, int variant, void* workspace,
                                        size_t workspace_bytes, hipEvent_t* events,
                                        int n_events, int* n_kernels, hipStream_t stream) {
  size_t tb = 0;
  sana_status_t s = sana::check_shape(B, N, H, d, dtype, &tb);
  if (s != SANA_OK) return s;
  if (variant != SANA_VARIANT_AUTO && variant != SANA_VARIANT_SPLIT && variant != SANA_VARIANT_FUSED)
    return SANA_ERR_UNSUPPORTED;
  const sana::Plan p = sana::make_plan(B, N, H);
  const bool fused = sana::use_fused(p, variant);
  const int nk = fused ? 1 : 3;
  if (n_kernels) *n_kernels = nk;
  if (!events || n_events < nk + 1) return SANA_ERR_INVALID_ARG;
  for (int i = 0; i <= nk; ++i)
    if (!events[i]) return SANA_ERR_INVALID_ARG;
  if (!q || !k || !v || !out) return SANA_ERR_INVALID_ARG;
  if ((s = sana::check_eps(eps)) != SANA_OK) return s;
  if (sana::misaligned(q) || sana::misaligned(k) || sana::misaligned(v) || sana::misaligned(out))
    return SANA_ERR_ALIGNMENT;
  if (sana::overlaps(out, tb, q, tb) || sana::overlaps(out, tb, k, tb) ||
      sana::overlaps(out, tb, v, tb))
    return SANA_ERR_INVALID_ARG;
  if ((s = sana::check_workspace(p, workspace, workspace_bytes)) != SANA_OK) return s;
  if (sana::overlaps(out, tb, workspace, p.workspace_bytes)) return SANA_ERR_INVALID_ARG;

  (void)hipGetLastError();
  if (hipEventRecord(events[0], stream) != hipSuccess) return SANA_ERR_HIP;
  if (fused) {
    if (sana::launch_fused(p, dtype, q, k, v, out, eps, stream) != hipSuccess) return SANA_ERR_HIP;
    return sana::to_status(hipEventRecord(events[1], stream));
  }
  float* partials = static_cast<float*>(workspace);
  float* state = reinterpret_cast<float*>(static_cast<char*>(workspace) + p.partial_bytes);
  if (sana::launch_reduce(p, dtype, k, v, partials, stream) != hipSuccess) return SANA_ERR_HIP;
  if (hipEventRecord(events[1], stream) != hipSuccess) return SANA_ERR_HIP;
  if (sana::launch_combine(p, partials, state, stream) != hipSuccess) return SANA_ERR_HIP;
  if (hipEventRecord(events[2], stream) != hipSuccess) return SANA_ERR_HIP;
  if (sana::launch_apply(p, dtype, q, state, out, eps, stream) != hipSuccess) return SANA_ERR_HIP;
  return sana::to_status(hipEventRecord(events[3], stream));
}

sana_status_t sana_linattn_fwd(const void* q, const void* k, const void* v, void* out, int64_t B,
                               int64_t N, int64_t H, int64_t d, float eps, int dtype,
                               void* workspace, size_t workspace_bytes, hipStream_t stream) {
  return sana_linattn_fwd_variant(q, k, v, out, B, N, H, d, eps, dtype, SANA_VARIANT_AUTO,
                                  workspace, workspace_bytes, stream);
}

sana_status_t sana_linattn_kv_state(const void* k, const void* v, float* state, int64_t B,
                                    int64_t N, int64_t H, int64_t d, int dtype, void* workspace,
                                    size_t workspace_bytes, hipStream_t stream) {
  size_t tb = 0;
  sana_status_t s = sana::check_shape(B, N, H, d, dtype, &tb);
  if (s != SANA_OK) return s;
  if (!k || !v || !state) return SANA_ERR_INVALID_ARG;
  if (sana::misaligned(k) || sana::misaligned(v) || sana::misaligned(state))
    return SANA_ERR_ALIGNMENT;
  const Plan p = sana::make_plan(B, N, H);
  if ((s = sana::check_workspace(p, workspace, workspace_bytes)) != SANA_OK) return s;
  const size_t sb = static_cast<size_t>(B * H) * sana::kStateFloats * 4;
  if (sana::overlaps(state, sb, k, tb) || sana::overlaps(state, sb, v, tb) ||
      sana::overlaps(state, sb, workspace, p.partial_bytes))
    return SANA_ERR_INVALID_ARG;
  (void)hipGetLastError();
  return sana::run_state(p, dtype, k, v, state, workspace, stream);
}

sana_status_t sana_linattn_apply(const void* q, const float* state, void* out, int64_t B,
                                 int64_t N, int64_t H, int64_t d, float eps, int dtype,
                                 hipStream_t stream) {
  size_t tb = 0;
  sana_status_t s = sana::check_shape(B, N, H, d, dtype, &tb);
  if (s != SANA_OK) return s;
  if (!q || !state || !out) return SANA_ERR_INVALID_ARG;
  if ((s = sana::check_eps(eps)) != SANA_OK) return s;
  if (sana::misaligned(q) || sana::misaligned(state) || sana::misaligned(out))
    return SANA_ERR_ALIGNMENT;
  const size_t sb = static_cast<size_t>(B * H) * sana::kStateFloats * 4;
  if (sana::overlaps(out, tb, q, tb) || sana::overlaps(out, tb, state, sb))
    return SANA_ERR_INVALID_ARG;
  const Plan p = sana::make_plan(B, N, H);
  (void)hipGetLastError();
  return sana::to_status(sana::launch_apply(p, dtype, q, state, out, eps, stream));
}

const char* sana_linattn_strerror(int status) {
  switch (status) {
    case SANA_OK: return "success";
    case SANA_ERR_INVALID_ARG: return "invalid argument";
    case SANA_ERR_UNSUPPORTED: return "unsupported head dim, dtype or variant";
    case SANA_ERR_WORKSPACE: return "workspace missing or too small";
    case SANA_ERR_ALIGNMENT: return "pointer not aligned (tensors 16 bytes, workspace 256 bytes)";
    case SANA_ERR_HIP: return "HIP kernel launch failed";
    default: return "unknown status";
  }
}

int sana_linattn_version(void) { return SANA_LINATTN_VERSION; }

}  // extern "C"
