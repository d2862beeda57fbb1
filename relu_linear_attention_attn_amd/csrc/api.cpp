// C ABI of the ReLU linear self-attention forward pass (include/sana_linattn.h):
// argument checks, the work split, workspace layout and kernel launches.
// Every check runs on the host before the first HIP call.

#include "sana_linattn.h"

#include <cmath>
#include <cstdint>
#include <cstdlib>
#include <cstring>
#include <algorithm>
#include <atomic>
#include <mutex>

#include "linattn_internal.h"

namespace sana {
namespace {

constexpr int64_t kMinReduceChunk = 256;       // tokens: 8 tiles per wave at 2 sub-streams
constexpr int64_t kMinApplyChunk = 256;
constexpr int64_t kWorkspaceBlocks = 4096;     // reduction blocks the workspace allows for
constexpr int64_t kMaxReduceChunks = 64;
constexpr int64_t kMaxRounds = 4;              // block rounds considered when fitting the grid
constexpr int64_t kFusedMaxN = 1024;           // AUTO picks the fused kernel up to this N
constexpr int64_t kReduceWavesPerCu = 8;
constexpr size_t kAlign = 256;

int64_t cdiv(int64_t a, int64_t b) { return (a + b - 1) / b; }

// Tokens per chunk for `chunks` chunks of N, in whole tiles. An even tile
// count is made odd: chunk starts then do not share the high power-of-two
// alignment that would send every chunk's stream to the same HBM channels.
int64_t chunk_tokens(int64_t N, int64_t chunks) {
  int64_t tiles = cdiv(cdiv(N, chunks), kTile);
  if (tiles > 1 && tiles % 2 == 0) ++tiles;
  return tiles * kTile;
}
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
  // The workspace holds up to red_chunks_max chunk partials per head. The
  // bound stops depending on N once N >= kMinReduceChunk * red_chunks_max.
  p.red_chunks_max = clamp64(std::min(cdiv(kWorkspaceBlocks, p.units), cdiv(N, kMinReduceChunk)),
                             1, kMaxReduceChunks);
  p.red_chunk = chunk_tokens(N, p.red_chunks_max);
  p.red_chunks = cdiv(N, p.red_chunk);
  p.app_chunk = cdiv(N, kTile) * kTile;
  p.app_chunks = 1;
  const size_t bh = static_cast<size_t>(B * H);
  p.partial_bytes = align_up(static_cast<size_t>(p.red_chunks_max) * bh * kStateFloats * 4);
  p.state_bytes = align_up(bh * kStateFloats * 4);
  p.ctl_bytes = align_up(static_cast<size_t>(p.units) * sizeof(unsigned long long));
  p.workspace_bytes = p.partial_bytes + p.state_bytes + p.ctl_bytes;
  return p;
}

namespace {

struct DeviceCaps {
  int cus = 0;
  int occ[2][2] = {{1, 1}, {1, 1}};  // [kernel: reduce, apply][dtype]
};

const DeviceCaps& device_caps() {
  constexpr int kMaxDevices = 64;
  static DeviceCaps caps[kMaxDevices];
  static std::once_flag once[kMaxDevices];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) dev = 0;
  std::call_once(once[dev], [dev] {
    DeviceCaps c;
    if (hipDeviceGetAttribute(&c.cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
        c.cus <= 0)
      c.cus = 256;
    for (int dt = 0; dt < 2; ++dt) {
      c.occ[0][dt] = occupancy_blocks_per_cu(KernelKind::kReduce, dt);
      c.occ[1][dt] = occupancy_blocks_per_cu(KernelKind::kApply, dt);
    }
    caps[dev] = c;
  });
  return caps[dev];
}

// Chunks per unit such that the grid (units * chunks blocks) fills whole
// rounds of `cap` co-resident blocks as closely as possible.
int64_t pick_chunks(int64_t units, int64_t cap, int64_t max_chunks) {
  int64_t best = 1;
  double best_fill = -1.0;
  for (int64_t k = 1; k <= kMaxRounds; ++k) {
    const int64_t c = clamp64(k * cap / units, 1, max_chunks);
    const int64_t blocks = units * c;
    const int64_t rounds = cdiv(blocks, cap);
    const double fill = static_cast<double>(blocks) / static_cast<double>(rounds * cap);
    if (fill > best_fill + 0.01) {
      best_fill = fill;
      best = c;
    }
  }
  return best;
}

}  // namespace

void fit_plan_to_device(Plan& p, int dtype) {
  const DeviceCaps& c = device_caps();
  const int dt = dtype == SANA_DTYPE_BF16 ? 1 : 0;
  const int64_t rcap = static_cast<int64_t>(c.cus) * c.occ[0][dt];
  const int64_t acap = static_cast<int64_t>(c.cus) * c.occ[1][dt];
  // The reduction's cost grows with its chunk count (every chunk adds a
  // partial to write and fold), so it takes the fewest chunks that still
  // keep about kReduceWavesPerCu waves streaming on every CU, within one
  // round of co-resident blocks.
  const int64_t waves = static_cast<int64_t>(c.cus) * kReduceWavesPerCu;
  const int64_t want = cdiv(waves, p.units * reduce_block_waves(dtype));
  int64_t rc = clamp64(std::min(want, std::max<int64_t>(1, rcap / p.units)), 1, p.red_chunks_max);
#ifdef SANA_TUNING
  if (const char* e = getenv("SANA_RED_CHUNKS")) rc = clamp64(atoll(e), 1, p.red_chunks_max);
#endif
  p.red_chunk = chunk_tokens(p.N, rc);
  p.red_chunks = cdiv(p.N, p.red_chunk);
  int64_t ac = pick_chunks(p.units, acap, std::max<int64_t>(1, cdiv(p.N, kMinApplyChunk)));
#ifdef SANA_TUNING
  if (const char* e = getenv("SANA_APP_CHUNKS")) ac = std::max<int64_t>(1, atoll(e));
#endif
  p.app_chunk = chunk_tokens(p.N, ac);
  p.app_chunks = cdiv(p.N, p.app_chunk);
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

// A fresh tag per call for the per-pair control words (48 bits; never 0).
unsigned long long next_epoch() {
  static std::atomic<unsigned long long> counter{0};
  unsigned long long e;
  do {
    e = (counter.fetch_add(1, std::memory_order_relaxed) + 1) & ((1ull << 48) - 1);
  } while (e == 0);
  return e;
}

struct WorkspaceParts {
  float* partials;
  float* state;
  unsigned long long* ctl;
};

WorkspaceParts split_workspace(const Plan& p, void* ws) {
  char* base = static_cast<char*>(ws);
  return {reinterpret_cast<float*>(base), reinterpret_cast<float*>(base + p.partial_bytes),
          reinterpret_cast<unsigned long long*>(base + p.partial_bytes + p.state_bytes)};
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
  Plan fp = p;
  sana::fit_plan_to_device(fp, dtype);
  if (sana::use_fused(fp, variant))
    return sana::to_status(sana::launch_fused(fp, dtype, q, k, v, out, eps, stream));
  const sana::WorkspaceParts w = sana::split_workspace(fp, workspace);
  if (sana::launch_reduce(fp, dtype, k, v, w.partials, w.state, w.ctl, sana::next_epoch(),
                          stream) != hipSuccess)
    return SANA_ERR_HIP;
  return sana::to_status(sana::launch_apply(fp, dtype, q, w.state, out, eps, stream));
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
  const int nk = fused ? 1 : 2;
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
  Plan fp = p;
  sana::fit_plan_to_device(fp, dtype);
  if (hipEventRecord(events[0], stream) != hipSuccess) return SANA_ERR_HIP;
  if (fused) {
    if (sana::launch_fused(fp, dtype, q, k, v, out, eps, stream) != hipSuccess) return SANA_ERR_HIP;
    return sana::to_status(hipEventRecord(events[1], stream));
  }
  const sana::WorkspaceParts w = sana::split_workspace(fp, workspace);
  if (sana::launch_reduce(fp, dtype, k, v, w.partials, w.state, w.ctl, sana::next_epoch(),
                          stream) != hipSuccess)
    return SANA_ERR_HIP;
  if (hipEventRecord(events[1], stream) != hipSuccess) return SANA_ERR_HIP;
  if (sana::launch_apply(fp, dtype, q, w.state, out, eps, stream) != hipSuccess) return SANA_ERR_HIP;
  return sana::to_status(hipEventRecord(events[2], stream));
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
      sana::overlaps(state, sb, workspace, p.workspace_bytes))
    return SANA_ERR_INVALID_ARG;
  (void)hipGetLastError();
  Plan fp = p;
  sana::fit_plan_to_device(fp, dtype);
  const sana::WorkspaceParts w = sana::split_workspace(fp, workspace);
  return sana::to_status(sana::launch_reduce(fp, dtype, k, v, w.partials, state, w.ctl,
                                             sana::next_epoch(), stream));
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
  Plan p = sana::make_plan(B, N, H);
  (void)hipGetLastError();
  sana::fit_plan_to_device(p, dtype);
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
