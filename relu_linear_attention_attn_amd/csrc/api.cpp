// C ABI of the ReLU linear self-attention forward pass (include/sana_linattn.h):
// argument checks, the work split, workspace layout and kernel launches.
// Every check runs on the host before the first HIP call.

#include "sana_linattn.h"

#include <climits>
#include <cmath>
#include <cstdint>
#include <cstdlib>
#include <cstdio>
#include <cstring>
#include <algorithm>
#include <atomic>
#include <chrono>
#include <random>
#include <mutex>

#include "linattn_internal.h"

namespace sana {
namespace {

constexpr int64_t kMinReduceChunk = 256;       // tokens: 8 tiles per wave at 2 sub-streams
constexpr int64_t kMinApplyChunk = 256;
constexpr int64_t kChunkCostTokens = 64;       // a (unit, chunk) block's fixed cost, in tokens
constexpr int64_t kMaxChunkRounds = 8;         // rounds the chunk search looks at
constexpr int64_t kMaxUnits = int64_t(1) << 22;  // head pairs per call; also the largest
                                                 // searched (unit, chunk) grid
constexpr int64_t kWorkspaceBlocks = 4096;     // reduction blocks the workspace allows for
constexpr int64_t kMaxReduceChunks = 64;
constexpr int64_t kFusedMaxN = 1024;           // AUTO picks the fused kernel up to this N
constexpr int64_t kReduceWavesPerCu = 8;
constexpr int64_t kMaxRangeBlocks = 2048;      // bf16 blocks per launch, any device
constexpr int64_t kMinTilesPerWave = 4;        // bf16: fewer tiles per wave than this
                                               // and blocks are not worth their epilogue
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
  // head pairs: no grid has more blocks than max(kMaxUnits, 16 x the
  // co-resident blocks), so every launch stays within 2^32 work-items; the
  // state and workspace sizes stay far below the tensor limit then
  int64_t units = 0;
  if (__builtin_mul_overflow(B, cdiv(H, kHeadsPerBlock), &units) || units > kMaxUnits)
    return SANA_ERR_INVALID_ARG;
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
  p.ld = H * kHeadDim;
  p.pairs = cdiv(H, kHeadsPerBlock);
  p.units = B * p.pairs;
  p.tiles = cdiv(N, kTile);
  const int64_t F = p.units * p.tiles;
  // bf16 ranges: at most kMaxRangeBlocks blocks, so at least ceil(F / that)
  // tiles per block and at most ceil(T / q_min) + 1 blocks touching a unit.
  const int64_t q_min = cdiv(F, kMaxRangeBlocks);
  // slots: enough for balanced ranges and for a one-round (unit, chunk) grid
  // of at most kMaxRangeBlocks blocks
  p.slots = std::max(std::min(p.tiles, cdiv(p.tiles, q_min)) + 1,
                     std::min(p.tiles, std::max<int64_t>(1, kMaxRangeBlocks / p.units)));
  p.red_q = q_min;
  p.red_blocks = cdiv(F, q_min);
  p.red_cb = 0;
  p.red_cq = 0;
  // fp32 chunks: at most red_chunks_max, a bound that stops depending on N
  // once N >= kMinReduceChunk * red_chunks_max.
  p.red_chunks_max = clamp64(std::min(cdiv(kWorkspaceBlocks, p.units), cdiv(N, kMinReduceChunk)),
                             1, kMaxReduceChunks);
  p.red_chunk = chunk_tokens(N, p.red_chunks_max);
  p.red_chunks = cdiv(N, p.red_chunk);
  p.app_chunk = cdiv(N, kTile) * kTile;
  p.app_chunks = 1;
  p.app_q = 0;
  p.app_blocks = 0;
  const size_t bh = static_cast<size_t>(B * H);
  const size_t f32_partials = static_cast<size_t>(p.red_chunks_max) * bh * kStateFloats * 4;
  const size_t bf16_partials =
      static_cast<size_t>(p.units) * static_cast<size_t>(p.slots) * 2 * kStateFloats * 4;
  p.partial_bytes = align_up(std::max(f32_partials, bf16_partials));
  p.bf16_partial_bytes = align_up(bf16_partials);
  p.state_bytes = align_up(bh * kStateFloats * 4);
  p.ctl_bytes = align_up(static_cast<size_t>(p.units) * sizeof(unsigned long long));
  p.workspace_bytes = p.partial_bytes + p.state_bytes + p.ctl_bytes;
  return p;
}

namespace {

struct DeviceCaps {
  int cus = 0;
  int occ[2][2] = {{1, 1}, {1, 1}};  // [kernel: reduce, apply][dtype]
  int occ_bwd_kv = 1;                // backward k/v pass (bf16)
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
    c.occ_bwd_kv = occupancy_blocks_per_cu(KernelKind::kBwdKV, 1);
    caps[dev] = c;
  });
  return caps[dev];
}

}  // namespace

// Chunks per unit for a (unit, chunk) grid on `slots` co-resident blocks.
// One round when the units fit it and fill at least 3/4 of the slots
// (measured: the idle rest costs less than an extra round, since fewer
// blocks each stream faster); otherwise the count that minimises the
// modelled time, rounds of blocks times one block's tokens plus a fixed
// per-block cost, so that a grid that would leave many slots idle is cut
// into more, shorter chunks.
int64_t grid_chunks(int64_t units, int64_t N, int64_t slots) {
  const int64_t max_c = std::max<int64_t>(1, cdiv(N, kMinApplyChunk));
  const int64_t one = clamp64(slots / units, 1, max_c);
  if (units <= slots && 4 * units * cdiv(N, chunk_tokens(N, one)) >= 3 * slots) return one;
  const int64_t last = std::min(max_c, kMaxChunkRounds * cdiv(slots, units));
  int64_t best = 1, best_t = INT64_MAX;
  for (int64_t c = 1; c <= last; ++c) {
    const int64_t chunk = chunk_tokens(N, c);
    const int64_t items = units * cdiv(N, chunk);
    if (c > 1 && items > kMaxUnits) break;
    const int64_t t = cdiv(items, slots) * (chunk + kChunkCostTokens);
    if (t < best_t) best_t = t, best = c;
  }
  return best;
}

void fit_plan_to_device(Plan& p, int dtype) {
  const DeviceCaps& c = device_caps();
  const int dt = dtype == SANA_DTYPE_BF16 ? 1 : 0;
  const int64_t rcap = static_cast<int64_t>(c.cus) * c.occ[0][dt];
  const int64_t acap = static_cast<int64_t>(c.cus) * c.occ[1][dt];
  if (dt == 1) {
    // bf16 reduction: balanced ranges, one round of co-resident blocks over
    // equal shares of the (unit, tile) index; never more blocks than the
    // workspace allows for
    const int64_t F = p.units * p.tiles;
    int64_t g = std::min<int64_t>(rcap, kMaxRangeBlocks);
    g = std::min(g, std::max<int64_t>(1, F / (block_waves(KernelKind::kReduce, dt) *
                                                 kMinTilesPerWave)));
    p.red_q = cdiv(F, g);
    p.red_blocks = cdiv(F, p.red_q);
    // ... unless a (unit, chunk) grid fills at least 3/4 of that round: its
    // blocks all start at the same token offsets of their head pairs and
    // advance together, so the head pairs of a token row are read close in
    // time (measured: the reduce pattern at 6.95 TB/s over 210 such blocks,
    // against 6.2 TB/s over 256 balanced ranges, whose blocks sit at
    // scattered offsets)
    const int64_t cap = std::min<int64_t>(rcap, kMaxRangeBlocks);
    const int64_t cq = chunk_tokens(p.N, grid_chunks(p.units, p.N, cap)) / kTile;
    const int64_t cb = cdiv(p.tiles, cq);
    if (p.units * cb <= cap && 4 * p.units * cb >= 3 * cap && cb <= p.slots) {
      p.red_cb = cb;
      p.red_cq = cq;
    }
  } else {
    // fp32 reduction: (unit, chunk) grid with the fewest chunks that keep
    // about kReduceWavesPerCu waves streaming per CU within one round
    const int64_t waves = static_cast<int64_t>(c.cus) * kReduceWavesPerCu;
    const int64_t want = cdiv(waves, p.units * block_waves(KernelKind::kReduce, dtype));
    int64_t rc = clamp64(std::min(want, std::max<int64_t>(1, rcap / p.units)), 1,
                         p.red_chunks_max);
    p.red_chunk = chunk_tokens(p.N, rc);
    p.red_chunks = cdiv(p.N, p.red_chunk);
  }
  // apply and backward k/v pass: (unit, chunk) grids, each for its kernel's
  // occupancy
  int64_t ac = grid_chunks(p.units, p.N, acap);
  p.app_chunk = chunk_tokens(p.N, ac);
  p.app_chunks = cdiv(p.N, p.app_chunk);
  // more head pairs than co-resident apply blocks: the (unit, chunk) grid
  // would need several rounds, the last one part empty; balanced ranges over
  // one round keep every CU streaming to the end (bf16)
  if (dt == 1 && p.units > acap) {
    const int64_t F = p.units * p.tiles;
    const int64_t g = std::max<int64_t>(
        1, std::min(std::min<int64_t>(acap, kMaxRangeBlocks),
                    F / (block_waves(KernelKind::kApply, dt) * kMinTilesPerWave)));
    p.app_q = cdiv(F, g);
    p.app_blocks = cdiv(F, p.app_q);
  }
  int64_t bc = grid_chunks(p.units, p.N, static_cast<int64_t>(c.cus) * c.occ_bwd_kv);
  p.bkv_chunk = chunk_tokens(p.N, bc);
  p.bkv_chunks = cdiv(p.N, p.bkv_chunk);
}

namespace {

sana_status_t check_workspace(const Plan& p, const void* ws, size_t ws_bytes) {
  if (p.workspace_bytes == 0) return SANA_OK;
  if (!ws || ws_bytes < p.workspace_bytes) return SANA_ERR_WORKSPACE;
  if ((reinterpret_cast<uintptr_t>(ws) & (kAlign - 1)) != 0) return SANA_ERR_ALIGNMENT;
  return SANA_OK;
}

sana_status_t to_status(hipError_t e) { return e == hipSuccess ? SANA_OK : SANA_ERR_HIP; }

constexpr int kBwdKernels = 3;

// Backward workspace (bf16): the forward reduction's partials, then bwd_q's.
size_t bwd_workspace_bytes(const Plan& p) { return 2 * p.bf16_partial_bytes; }

bool valid_variant(int variant) {
  return variant == SANA_VARIANT_AUTO || variant == SANA_VARIANT_SPLIT ||
         variant == SANA_VARIANT_FUSED;
}

// The kernel arrangement a call runs. AUTO, for sequences up to kFusedMaxN
// tokens (beyond, the split pair), the fused kernel (one block per head
// pair over all N tokens: one launch, no partials) when
//  * the call is tiny (units x N <= kTinyUnitTokens), or
//  * N <= kFusedMaxN / 2 (a block's whole unit is short), or
//  * units x N >= (CUs / 2) x kFusedMaxN (enough pairs that the fused grid
//    keeps the device streaming),
// else the split pair. Measured, split / fused us (256 CUs): N = 1024 with
// 36 pairs 14.7 / 15.7, 48 pairs 14.3 / 19.0, 64 pairs 15.2 / 19.3, 96 pairs
// 19.7 / 21.2, 128 pairs 21.5 / 21.5, 280 pairs 39.2 / 36.5, 560 pairs 65.9 /
// 57.9; N = 512 with 36 pairs 14.0 / 10.7; N = 256 with 140 pairs 15.7 /
// 8.1. Running the fused kernel over whole rounds of head pairs and the
// split pair over the rest measured slower (16 x 1024 x 70: 63.9 against
// 61.1 us with one fused block per CU): the short last fused round costs
// less than two more launches over its units.
// Queries the device's CU count once per device.
constexpr int64_t kTinyUnitTokens = 4096;  // units x N at or below which one launch wins

int resolve_variant(const Plan& p, int dtype, int variant) {
  (void)dtype;
  if (variant != SANA_VARIANT_AUTO) return variant;
  if (p.N > kFusedMaxN) return SANA_VARIANT_SPLIT;
  if (p.units * p.N <= kTinyUnitTokens || 2 * p.N <= kFusedMaxN) return SANA_VARIANT_FUSED;
  const int64_t cus = device_caps().cus;
  return 2 * p.units * p.N >= cus * kFusedMaxN ? SANA_VARIANT_FUSED : SANA_VARIANT_SPLIT;
}

int kernels_of(int variant) { return variant == SANA_VARIANT_SPLIT ? 2 : 1; }

// A fresh tag per call for the per-pair control words (48 bits; never 0).
// The count starts at a per-process random value, so a control word left in
// a reused workspace by another process or another copy of the library is
// unlikely to carry the tag of a call here.
unsigned long long next_epoch() {
  static std::atomic<unsigned long long> counter{[] {
    std::random_device rd;
    return (static_cast<unsigned long long>(rd()) << 32) ^ rd() ^
           static_cast<unsigned long long>(
               std::chrono::steady_clock::now().time_since_epoch().count());
  }()};
  unsigned long long e;
  do {
    e = (counter.fetch_add(1, std::memory_order_relaxed) + 1) & ((1ull << 48) - 1);
  } while (e == 0);
  return e;
}

struct WorkspaceParts {
  float* partials;
  float* state;
  unsigned long long* ctl;  // one control word per unit
};

WorkspaceParts split_workspace(const Plan& p, void* ws) {
  char* base = static_cast<char*>(ws);
  unsigned long long* ctl =
      reinterpret_cast<unsigned long long*>(base + p.partial_bytes + p.state_bytes);
  return {reinterpret_cast<float*>(base), reinterpret_cast<float*>(base + p.partial_bytes), ctl};
}

}  // namespace
}  // namespace sana

using sana::Plan;

extern "C" {

sana_status_t sana_linattn_workspace_size(int64_t B, int64_t N, int64_t H, int64_t d, sana_dtype_t dtype,
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

}  // extern "C"

namespace sana {
namespace {

bool valid_fmap(int fmap) {
  return fmap == SANA_FMAP_RELU || fmap == SANA_FMAP_ELU1 || fmap == SANA_FMAP_COS;
}

// Bytes a [B][N][H][d] input with token stride ld spans from its first
// element: (B N - 1) ld + H d elements. 0 when that overflows (or passes
// 2^62 bytes).
size_t strided_span(int64_t B, int64_t N, int64_t H, int64_t d, int64_t ld, int64_t item) {
  int64_t t = 0;
  if (__builtin_mul_overflow(B, N, &t) || __builtin_mul_overflow(t - 1, ld, &t) ||
      __builtin_add_overflow(t, H * d, &t) || __builtin_mul_overflow(t, item, &t) ||
      t >= (int64_t(1) << 62))
    return 0;
  return static_cast<size_t>(t);
}

// The forward pass behind every fwd entry point. events (may be NULL) are
// recorded before the first kernel and after each kernel. Feature maps
// other than ReLU, and q, k, v with a token stride ld other than H d, run
// the split kernels only (ld = 0 means H d).
// ws_source (may be NULL) supplies the workspace once every host check has
// passed, in place of workspace / workspace_bytes.
sana_status_t forward(const void* q, const void* k, const void* v, void* out, int64_t B,
                      int64_t N, int64_t H, int64_t d, float eps, int dtype, int variant,
                      void* workspace, size_t workspace_bytes, hipEvent_t* events, int n_events,
                      int* n_kernels, hipStream_t stream, int fmap = SANA_FMAP_RELU,
                      int64_t ld = 0, WorkspaceSource ws_source = nullptr) {
  size_t tb = 0;
  sana_status_t s = check_shape(B, N, H, d, dtype, &tb);
  if (s != SANA_OK) return s;
  if (!valid_variant(variant) || !valid_fmap(fmap)) return SANA_ERR_UNSUPPORTED;
  const int64_t item = dtype == SANA_DTYPE_F32 ? 4 : 2;
  if (ld == 0) ld = H * d;
  if (ld < H * d) return SANA_ERR_INVALID_ARG;
  const size_t in_bytes = strided_span(B, N, H, d, ld, item);
  if (in_bytes == 0) return SANA_ERR_INVALID_ARG;
  if ((ld * item) % 16 != 0) return SANA_ERR_ALIGNMENT;  // every token row 16-byte aligned
  const bool split_only = fmap != SANA_FMAP_RELU || ld != H * d;
  if (split_only && variant == SANA_VARIANT_FUSED) return SANA_ERR_UNSUPPORTED;
  if (split_only) variant = SANA_VARIANT_SPLIT;
  Plan p = make_plan(B, N, H);
  p.ld = ld;
  const int run = resolve_variant(p, dtype, variant);
  const int nk = kernels_of(run);
  if (n_kernels) *n_kernels = nk;
  if (events) {
    if (n_events < nk + 1) return SANA_ERR_INVALID_ARG;
    for (int i = 0; i <= nk; ++i)
      if (!events[i]) return SANA_ERR_INVALID_ARG;
  }
  if (!q || !k || !v || !out) return SANA_ERR_INVALID_ARG;
  if ((s = check_eps(eps)) != SANA_OK) return s;
  if (misaligned(q) || misaligned(k) || misaligned(v) || misaligned(out)) return SANA_ERR_ALIGNMENT;
  if (overlaps(out, tb, q, in_bytes) || overlaps(out, tb, k, in_bytes) ||
      overlaps(out, tb, v, in_bytes))
    return SANA_ERR_INVALID_ARG;
  if (ws_source && ws_source(&workspace, &workspace_bytes) != hipSuccess) return SANA_ERR_HIP;
  if ((s = check_workspace(p, workspace, workspace_bytes)) != SANA_OK) return s;
  // the reduction writes partials while other blocks still read k and v, and
  // the apply writes out: the workspace may alias no tensor
  if (overlaps(out, tb, workspace, p.workspace_bytes) ||
      overlaps(workspace, p.workspace_bytes, q, in_bytes) ||
      overlaps(workspace, p.workspace_bytes, k, in_bytes) ||
      overlaps(workspace, p.workspace_bytes, v, in_bytes))
    return SANA_ERR_INVALID_ARG;

  // every check passed: from here on HIP is called
  (void)hipGetLastError();  // clear an unrelated earlier error
  Plan fp = p;
  fit_plan_to_device(fp, dtype);
  auto mark = [&](int i) { return !events || hipEventRecord(events[i], stream) == hipSuccess; };
  if (!mark(0)) return SANA_ERR_HIP;
  const WorkspaceParts w = split_workspace(fp, workspace);
  if (run == SANA_VARIANT_FUSED) {
    if (launch_fused(fp, dtype, device_caps().cus, q, k, v, out, eps, stream) != hipSuccess)
      return SANA_ERR_HIP;
    return mark(1) ? SANA_OK : SANA_ERR_HIP;
  }
  // split: bf16 hands the reduction's partials straight to the apply (no
  // fold at the end of the reduction); fp32 folds, then applies the state
  const bool bf16 = dtype == SANA_DTYPE_BF16;
  if (launch_reduce(fp, dtype, !bf16, k, v, w.partials, w.state, w.ctl, next_epoch(), stream,
                    fmap) != hipSuccess)
    return SANA_ERR_HIP;
  if (!mark(1)) return SANA_ERR_HIP;
  const hipError_t e = bf16 ? launch_apply_partials(fp, q, w.partials, out, eps, stream, fmap)
                            : launch_apply(fp, dtype, q, w.state, out, eps, stream, fmap);
  if (e != hipSuccess) return SANA_ERR_HIP;
  return mark(2) ? SANA_OK : SANA_ERR_HIP;
}

// Block-causal attention (blocks of L tokens): the plan treats each block
// as a batch item; the workspace holds that plan's parts and the prefix
// states.
struct BlockCausalPlan {
  Plan p;               // batch items = the B * F blocks of L tokens
  int64_t F;            // blocks per batch item
  size_t prefix_bytes;  // [B * F][H][d][d+1] fp32
  size_t workspace_bytes;
};

sana_status_t plan_block_causal(int64_t B, int64_t N, int64_t H, int64_t d, int64_t L,
                                int dtype, BlockCausalPlan* bc, size_t* tensor_bytes) {
  sana_status_t s = check_shape(B, N, H, d, dtype, tensor_bytes);
  if (s != SANA_OK) return s;
  if (L < 1 || N % L != 0) return SANA_ERR_INVALID_ARG;
  const int64_t F = N / L;
  // the blocks as batch items: B * F < 2^62 since B * N * H * d is
  if ((s = check_shape(B * F, L, H, d, dtype, nullptr)) != SANA_OK) return s;
  if (scan_grid_threads(B, cdiv(H, kHeadsPerBlock)) > UINT32_MAX) return SANA_ERR_INVALID_ARG;
  bc->p = make_plan(B * F, L, H);
  bc->F = F;
  bc->prefix_bytes = align_up(static_cast<size_t>(B * F * H) * kStateFloats * 4);
  bc->workspace_bytes = bc->p.workspace_bytes + bc->prefix_bytes;
  return SANA_OK;
}

// events (may be NULL) are recorded before the first kernel and after each of
// the three (reduction, scan, apply).
sana_status_t block_causal(const void* q, const void* k, const void* v, void* out, int64_t B,
                           int64_t N, int64_t H, int64_t d, int64_t L, float eps, int dtype,
                           void* workspace, size_t workspace_bytes, hipEvent_t* events,
                           int n_events, hipStream_t stream) {
  BlockCausalPlan bc;
  size_t tb = 0;
  sana_status_t s = plan_block_causal(B, N, H, d, L, dtype, &bc, &tb);
  if (s != SANA_OK) return s;
  if (events) {
    if (n_events < 4) return SANA_ERR_INVALID_ARG;
    for (int i = 0; i < 4; ++i)
      if (!events[i]) return SANA_ERR_INVALID_ARG;
  }
  if (!q || !k || !v || !out) return SANA_ERR_INVALID_ARG;
  if ((s = check_eps(eps)) != SANA_OK) return s;
  if (misaligned(q) || misaligned(k) || misaligned(v) || misaligned(out)) return SANA_ERR_ALIGNMENT;
  if (overlaps(out, tb, q, tb) || overlaps(out, tb, k, tb) || overlaps(out, tb, v, tb))
    return SANA_ERR_INVALID_ARG;
  if (!workspace || workspace_bytes < bc.workspace_bytes) return SANA_ERR_WORKSPACE;
  if ((reinterpret_cast<uintptr_t>(workspace) & (kAlign - 1)) != 0) return SANA_ERR_ALIGNMENT;
  for (const void* t : {static_cast<const void*>(out), q, k, v})
    if (overlaps(t, tb, workspace, bc.workspace_bytes)) return SANA_ERR_INVALID_ARG;

  (void)hipGetLastError();
  Plan fp = bc.p;
  fit_plan_to_device(fp, dtype);
  const WorkspaceParts w = split_workspace(fp, workspace);
  float* prefix = reinterpret_cast<float*>(static_cast<char*>(workspace) + fp.workspace_bytes);
  auto mark = [&](int i) { return !events || hipEventRecord(events[i], stream) == hipSuccess; };
  const bool bf16 = dtype == SANA_DTYPE_BF16;
  if (!mark(0)) return SANA_ERR_HIP;
  if (launch_reduce(fp, dtype, !bf16, k, v, w.partials, w.state, w.ctl, next_epoch(), stream) !=
      hipSuccess)
    return SANA_ERR_HIP;
  if (!mark(1)) return SANA_ERR_HIP;
  if (launch_scan_blocks(fp, dtype, bc.F, w.partials, w.state, prefix, stream) != hipSuccess)
    return SANA_ERR_HIP;
  if (!mark(2)) return SANA_ERR_HIP;
  if (launch_apply(fp, dtype, q, prefix, out, eps, stream) != hipSuccess) return SANA_ERR_HIP;
  return mark(3) ? SANA_OK : SANA_ERR_HIP;
}

// QKV projection + attention (bf16): sizes and checks shared by the size
// query and the call. x [B][N][C], w [3D][C], q and out [B][N][H][d].
struct QkvPlan {
  Plan p;                 // the attention's plan (apply grid)
  int64_t J;              // 256-token tiles per batch item: partial slots per head pair
  size_t x_bytes, w_bytes, t_bytes;  // x, w and q / out tensor bytes
  size_t workspace_bytes; // the partial states
};

// Token-causal attention: chunks per unit so that every unit's chunks make
// one round of kCausalWaves waves (the plan does not depend on the device).
sana_status_t plan_causal(int64_t B, int64_t N, int64_t H, int64_t d, int dtype, CausalPlan* cp,
                          size_t* tensor_bytes, int lg = 0, int64_t m = 0) {
  sana_status_t s = check_shape(B, N, H, d, dtype, tensor_bytes);
  if (s != SANA_OK) return s;
  if (dtype != SANA_DTYPE_BF16) return SANA_ERR_UNSUPPORTED;
  cp->lg = lg;
  cp->m = m;
  cp->B = B;
  cp->N = N;
  cp->H = H;
  cp->pairs = cdiv(H, 2);
  cp->units = B * cp->pairs;
  cp->tiles = cdiv(N, kTile);
  // about kCausalWaves waves in all (one block of 8 per CU) over chunks of
  // W tiles (rounding W to an odd count, as once tried, left the 4096px
  // latent with 245 blocks instead of 254 and the apply 8 us slower; chunks
  // of W and W + 1 tiles were 1 us slower than a short last chunk)
  const int64_t c = clamp64(kCausalWaves / cp->units, 1, std::min(cp->tiles, kMaxCausalChunks));
  cp->W = cdiv(cp->tiles, c);
  if (m > 1) cp->W = cdiv(cp->W, m) * m;  // chunks of whole blocks
  cp->chunks = cdiv(cp->tiles, cp->W);
  cp->parts_bytes =
      align_up(static_cast<size_t>(cp->units) * static_cast<size_t>(cp->chunks) * 2 * kStateFloats * 4);
  if (cdiv(cp->units * cp->chunks, 8) > INT32_MAX || cp->units * 2 * kStateFloats > INT64_C(1) << 40)
    return SANA_ERR_INVALID_ARG;
  return SANA_OK;
}

sana_status_t causal_forward(const void* q, const void* k, const void* v, void* out, int64_t B,
                             int64_t N, int64_t H, int64_t d, float eps, int dtype,
                             void* workspace, size_t workspace_bytes, hipEvent_t* events,
                             int n_events, hipStream_t stream, int lg = 0, int64_t m = 0) {
  CausalPlan cp;
  size_t tb = 0;
  sana_status_t s = plan_causal(B, N, H, d, dtype, &cp, &tb, lg, m);
  if (s != SANA_OK) return s;
  if (events) {
    if (n_events < 4) return SANA_ERR_INVALID_ARG;
    for (int i = 0; i < 4; ++i)
      if (!events[i]) return SANA_ERR_INVALID_ARG;
  }
  if (!q || !k || !v || !out) return SANA_ERR_INVALID_ARG;
  if ((s = check_eps(eps)) != SANA_OK) return s;
  if (misaligned(q) || misaligned(k) || misaligned(v) || misaligned(out)) return SANA_ERR_ALIGNMENT;
  if (overlaps(out, tb, q, tb) || overlaps(out, tb, k, tb) || overlaps(out, tb, v, tb))
    return SANA_ERR_INVALID_ARG;
  if (!workspace || workspace_bytes < cp.parts_bytes) return SANA_ERR_WORKSPACE;
  if ((reinterpret_cast<uintptr_t>(workspace) & (kAlign - 1)) != 0) return SANA_ERR_ALIGNMENT;
  for (const void* t : {static_cast<const void*>(out), q, k, v})
    if (overlaps(t, tb, workspace, cp.parts_bytes)) return SANA_ERR_INVALID_ARG;

  (void)hipGetLastError();
  float* parts = static_cast<float*>(workspace);
  auto mark = [&](int i) { return !events || hipEventRecord(events[i], stream) == hipSuccess; };
  if (!mark(0)) return SANA_ERR_HIP;
  if (launch_causal_states(cp, k, v, parts, stream) != hipSuccess) return SANA_ERR_HIP;
  if (!mark(1)) return SANA_ERR_HIP;
  if (launch_causal_scan(cp, parts, stream) != hipSuccess) return SANA_ERR_HIP;
  if (!mark(2)) return SANA_ERR_HIP;
  const hipError_t e = cp.m > 1 ? launch_causal_block_apply(cp, q, k, v, out, parts, eps, stream)
                                : launch_causal_apply(cp, q, k, v, out, parts, eps, stream);
  if (e != hipSuccess) return SANA_ERR_HIP;
  return mark(3) ? SANA_OK : SANA_ERR_HIP;
}

// Block-causal attention on the chunk-wise kernels (bf16), one state per
// chunk instead of one per block:
//   * blocks of 1, 2, 4, 8 or 16 tokens never straddle a tile, so every chunk
//     and tile boundary is a block boundary and the token-causal apply
//     computes them with its in-tile mask widened to whole blocks (lg);
//   * blocks of m = L / 16 whole tiles, chunks made of whole blocks: the
//     block-wise apply (each block's states first, then its queries).
// Longer blocks keep the per-block path, which is faster there: one state per
// block costs little once blocks are long, while chunks of whole long blocks
// leave too few waves (4096px latent, us per step, chunk-wise / per block:
// L = 64 178 / 584, 256 190 / 208, 512 222 / 163, 1024 220 / 141).
constexpr int64_t kMaxChunkedBlock = 256;  // tokens

struct ChunkedBlocks {
  bool on;
  int lg;
  int64_t m;
};

ChunkedBlocks chunked_blocks(int64_t L, int dtype) {
  if (dtype != SANA_DTYPE_BF16) return {false, 0, 0};
  for (int lg = 0; lg <= 4; ++lg)
    if (L == (int64_t(1) << lg)) return {true, lg, 0};
  if (L > kTile && L <= kMaxChunkedBlock && L % kTile == 0) return {true, 0, L / kTile};
  return {false, 0, 0};
}

sana_status_t block_causal_workspace(int64_t B, int64_t N, int64_t H, int64_t d, int64_t L,
                                     int dtype, size_t* bytes) {
  const ChunkedBlocks cb = chunked_blocks(L, dtype);
  if (cb.on) {
    CausalPlan cp;
    const sana_status_t s = plan_causal(B, N, H, d, dtype, &cp, nullptr, cb.lg, cb.m);
    if (s != SANA_OK) return s;
    if (N % L != 0) return SANA_ERR_INVALID_ARG;
    *bytes = cp.parts_bytes;
    return SANA_OK;
  }
  BlockCausalPlan bc;
  const sana_status_t s = plan_block_causal(B, N, H, d, L, dtype, &bc, nullptr);
  if (s != SANA_OK) return s;
  *bytes = bc.workspace_bytes;
  return SANA_OK;
}

sana_status_t block_causal_any(const void* q, const void* k, const void* v, void* out, int64_t B,
                               int64_t N, int64_t H, int64_t d, int64_t L, float eps, int dtype,
                               void* workspace, size_t workspace_bytes, hipEvent_t* events,
                               int n_events, hipStream_t stream) {
  const ChunkedBlocks cb = chunked_blocks(L, dtype);
  if (!cb.on)
    return block_causal(q, k, v, out, B, N, H, d, L, eps, dtype, workspace, workspace_bytes,
                        events, n_events, stream);
  CausalPlan cp;
  const sana_status_t s = plan_causal(B, N, H, d, dtype, &cp, nullptr, cb.lg, cb.m);
  if (s != SANA_OK) return s;
  if (N % L != 0) return SANA_ERR_INVALID_ARG;
  return causal_forward(q, k, v, out, B, N, H, d, eps, dtype, workspace, workspace_bytes, events,
                        n_events, stream, cb.lg, cb.m);
}

sana_status_t plan_qkv(int64_t B, int64_t N, int64_t C, int64_t H, int64_t d, QkvPlan* qp) {
  size_t tb = 0;
  sana_status_t s = check_shape(B, N, H, d, SANA_DTYPE_BF16, &tb);
  if (s != SANA_OK) return s;
  if (C < 1) return SANA_ERR_INVALID_ARG;
  if (C % 8 != 0) return SANA_ERR_UNSUPPORTED;  // 16-byte pieces of x and w rows
  // 32-bit offsets within a block's 256 x rows (and 64 W rows)
  if (C >= (int64_t(1) << 22)) return SANA_ERR_INVALID_ARG;
  int64_t xb = 0, wb = 0;
  if (__builtin_mul_overflow(B * N, C, &xb) || __builtin_mul_overflow(xb, int64_t(2), &xb) ||
      xb >= (int64_t(1) << 62))
    return SANA_ERR_INVALID_ARG;
  if (__builtin_mul_overflow(3 * H * d, C, &wb) || __builtin_mul_overflow(wb, int64_t(2), &wb) ||
      wb >= (int64_t(1) << 62))
    return SANA_ERR_INVALID_ARG;
  // the projection's grid (256 threads a block) within 2^32 work-items
  if (qkv_grid_blocks(B, N, H) > (int64_t(1) << 24)) return SANA_ERR_INVALID_ARG;
  qp->p = make_plan(B, N, H);
  qp->J = qkv_m_tiles(N);
  qp->x_bytes = static_cast<size_t>(xb);
  qp->w_bytes = static_cast<size_t>(wb);
  qp->t_bytes = tb;
  qp->workspace_bytes =
      align_up(static_cast<size_t>(qp->p.units * qp->J) * 2 * kStateFloats * 4);
  return SANA_OK;
}

constexpr int64_t kQkvGroupM = 8;  // token tiles per group of the projection's tile order

sana_status_t qkv_forward(const void* x, const void* w, void* q, void* out, int64_t B, int64_t N,
                          int64_t C, int64_t H, int64_t d, float eps, void* workspace,
                          size_t workspace_bytes, hipEvent_t* events, int n_events,
                          hipStream_t stream) {
  QkvPlan qp;
  sana_status_t s = plan_qkv(B, N, C, H, d, &qp);
  if (s != SANA_OK) return s;
  if (events) {
    if (n_events < 3) return SANA_ERR_INVALID_ARG;
    for (int i = 0; i < 3; ++i)
      if (!events[i]) return SANA_ERR_INVALID_ARG;
  }
  if (!x || !w || !q || !out) return SANA_ERR_INVALID_ARG;
  if ((s = check_eps(eps)) != SANA_OK) return s;
  if (misaligned(x) || misaligned(w) || misaligned(q) || misaligned(out)) return SANA_ERR_ALIGNMENT;
  const size_t tb = qp.t_bytes;
  if (overlaps(q, tb, x, qp.x_bytes) || overlaps(q, tb, w, qp.w_bytes) ||
      overlaps(out, tb, x, qp.x_bytes) || overlaps(out, tb, w, qp.w_bytes) ||
      overlaps(out, tb, q, tb))
    return SANA_ERR_INVALID_ARG;
  if (!workspace || workspace_bytes < qp.workspace_bytes) return SANA_ERR_WORKSPACE;
  if ((reinterpret_cast<uintptr_t>(workspace) & (kAlign - 1)) != 0) return SANA_ERR_ALIGNMENT;
  if (overlaps(workspace, qp.workspace_bytes, q, tb) ||
      overlaps(workspace, qp.workspace_bytes, out, tb) ||
      overlaps(workspace, qp.workspace_bytes, x, qp.x_bytes) ||
      overlaps(workspace, qp.workspace_bytes, w, qp.w_bytes))
    return SANA_ERR_INVALID_ARG;

  (void)hipGetLastError();
  Plan fp = qp.p;
  fit_plan_to_device(fp, SANA_DTYPE_BF16);
  int64_t gm = kQkvGroupM;
  float* partials = static_cast<float*>(workspace);
  auto mark = [&](int i) { return !events || hipEventRecord(events[i], stream) == hipSuccess; };
  if (!mark(0)) return SANA_ERR_HIP;
  if (launch_qkv_state(x, w, q, partials, B, N, C, H, gm, stream) != hipSuccess)
    return SANA_ERR_HIP;
  if (!mark(1)) return SANA_ERR_HIP;
  if (launch_apply_slots(fp, q, partials, qp.J, out, eps, stream) != hipSuccess)
    return SANA_ERR_HIP;
  return mark(2) ? SANA_OK : SANA_ERR_HIP;
}

// The backward pass (bf16): the forward state reduction (partials only),
// bwd_q (dq and the [dS | dz] partials), bwd_kv (dk, dv). events (may be
// NULL) are recorded before the first kernel and after each one. With a
// saved forward state (with_state: fp32 [B][H][d][d+1] of the same map), the
// reduction is skipped and bwd_q reads that state.
sana_status_t backward(const void* q, const void* k, const void* v, const void* g, void* dq,
                       void* dk, void* dv, int64_t B, int64_t N, int64_t H, int64_t d, float eps,
                       int dtype, void* workspace, size_t workspace_bytes, hipEvent_t* events,
                       int n_events, hipStream_t stream, int fmap = SANA_FMAP_RELU,
                       const float* state = nullptr, bool with_state = false) {
  size_t tb = 0;
  sana_status_t s = check_shape(B, N, H, d, dtype, &tb);
  if (s != SANA_OK) return s;
  if (dtype != SANA_DTYPE_BF16 || !valid_fmap(fmap)) return SANA_ERR_UNSUPPORTED;
  const int kernels = with_state ? kBwdKernels - 1 : kBwdKernels;
  if (events) {
    if (n_events < kernels + 1) return SANA_ERR_INVALID_ARG;
    for (int i = 0; i <= kernels; ++i)
      if (!events[i]) return SANA_ERR_INVALID_ARG;
  }
  if (with_state && !state) return SANA_ERR_INVALID_ARG;
  if (with_state && misaligned(state)) return SANA_ERR_ALIGNMENT;
  const size_t sbytes = static_cast<size_t>(B * H) * kStateFloats * 4;
  const void* in[] = {q, k, v, g};
  void* outs[] = {dq, dk, dv};
  for (const void* p : in)
    if (!p) return SANA_ERR_INVALID_ARG;
  for (const void* p : outs)
    if (!p) return SANA_ERR_INVALID_ARG;
  if ((s = check_eps(eps)) != SANA_OK) return s;
  for (const void* p : in)
    if (misaligned(p)) return SANA_ERR_ALIGNMENT;
  for (const void* p : outs)
    if (misaligned(p)) return SANA_ERR_ALIGNMENT;
  const Plan p = make_plan(B, N, H);
  const size_t wb = bwd_workspace_bytes(p);
  if (!workspace || workspace_bytes < wb) return SANA_ERR_WORKSPACE;
  if ((reinterpret_cast<uintptr_t>(workspace) & (kAlign - 1)) != 0) return SANA_ERR_ALIGNMENT;
  // an output may overlap nothing else (inputs may alias each other), and the
  // workspace no tensor
  for (const void* x : in)
    if (overlaps(workspace, wb, x, tb)) return SANA_ERR_INVALID_ARG;
  for (int i = 0; i < 3; ++i) {
    for (const void* x : in)
      if (overlaps(outs[i], tb, x, tb)) return SANA_ERR_INVALID_ARG;
    for (int j = i + 1; j < 3; ++j)
      if (overlaps(outs[i], tb, outs[j], tb)) return SANA_ERR_INVALID_ARG;
    if (overlaps(outs[i], tb, workspace, wb)) return SANA_ERR_INVALID_ARG;
    if (with_state && overlaps(outs[i], tb, state, sbytes)) return SANA_ERR_INVALID_ARG;
  }
  if (with_state && overlaps(workspace, wb, state, sbytes)) return SANA_ERR_INVALID_ARG;

  (void)hipGetLastError();
  Plan fp = p;
  fit_plan_to_device(fp, dtype);
  auto mark = [&](int i) { return !events || hipEventRecord(events[i], stream) == hipSuccess; };
  float* fwd_parts = static_cast<float*>(workspace);
  float* grad_parts =
      reinterpret_cast<float*>(static_cast<char*>(workspace) + fp.bf16_partial_bytes);
  if (!mark(0)) return SANA_ERR_HIP;
  if (with_state) {
    // k and v are read once, by the k/v pass
    if (launch_bwd_q(fp, q, g, dq, nullptr, state, grad_parts, eps, stream, fmap) != hipSuccess)
      return SANA_ERR_HIP;
    if (!mark(1)) return SANA_ERR_HIP;
    if (launch_bwd_kv(fp, k, v, dk, dv, grad_parts, stream, fmap) != hipSuccess)
      return SANA_ERR_HIP;
    return mark(2) ? SANA_OK : SANA_ERR_HIP;
  }
  // k and v are read again by the k/v pass after the q pass: the reduction
  // reads k with ordinary loads so that much of it is still in the Infinity
  // Cache then (2 x 16384 x 70 step 243 -> 230.6 us: reduction 47.7 -> 48.2
  // us, k/v pass 113.3 -> 100.2 us; keeping k and v both, 233 us: reduction
  // 53.0, k/v pass 97.7; v alone 232 us)
  if (launch_reduce(fp, dtype, false, k, v, fwd_parts, nullptr, nullptr, 0, stream, fmap,
                    true) != hipSuccess)
    return SANA_ERR_HIP;
  if (!mark(1)) return SANA_ERR_HIP;
  if (launch_bwd_q(fp, q, g, dq, fwd_parts, nullptr, grad_parts, eps, stream, fmap) !=
      hipSuccess)
    return SANA_ERR_HIP;
  if (!mark(2)) return SANA_ERR_HIP;
  if (launch_bwd_kv(fp, k, v, dk, dv, grad_parts, stream, fmap) != hipSuccess)
    return SANA_ERR_HIP;
  return mark(3) ? SANA_OK : SANA_ERR_HIP;
}

}  // namespace

sana_status_t forward_from_source(const void* q, const void* k, const void* v, void* out,
                                  int64_t B, int64_t N, int64_t H, int64_t d, float eps,
                                  int dtype, WorkspaceSource ws_source, hipStream_t stream) {
  return forward(q, k, v, out, B, N, H, d, eps, dtype, SANA_VARIANT_AUTO, nullptr, 0, nullptr, 0,
                 nullptr, stream, SANA_FMAP_RELU, 0, ws_source);
}

}  // namespace sana

extern "C" {

sana_status_t sana_linattn_fwd_variant(const void* q, const void* k, const void* v, void* out,
                                       int64_t B, int64_t N, int64_t H, int64_t d, float eps,
                                       sana_dtype_t dtype, sana_variant_t variant, void* workspace,
                                       size_t workspace_bytes, hipStream_t stream) {
  return sana::forward(q, k, v, out, B, N, H, d, eps, dtype, variant, workspace, workspace_bytes,
                       nullptr, 0, nullptr, stream);
}

sana_status_t sana_linattn_fwd_profiled(const void* q, const void* k, const void* v, void* out,
                                        int64_t B, int64_t N, int64_t H, int64_t d, float eps,
                                        sana_dtype_t dtype, sana_variant_t variant, void* workspace,
                                        size_t workspace_bytes, hipEvent_t* events,
                                        int n_events, int* n_kernels, hipStream_t stream) {
  if (!events) {
    if (n_kernels) {
      // still report the kernel count when the arguments allow it
      size_t tb = 0;
      if (sana::check_shape(B, N, H, d, dtype, &tb) == SANA_OK && sana::valid_variant(variant))
        *n_kernels =
            sana::kernels_of(sana::resolve_variant(sana::make_plan(B, N, H), dtype, variant));
    }
    return SANA_ERR_INVALID_ARG;
  }
  return sana::forward(q, k, v, out, B, N, H, d, eps, dtype, variant, workspace, workspace_bytes,
                       events, n_events, n_kernels, stream);
}

sana_status_t sana_linattn_fwd_fmap(const void* q, const void* k, const void* v, void* out,
                                    int64_t B, int64_t N, int64_t H, int64_t d, float eps,
                                    sana_dtype_t dtype, sana_fmap_t fmap, void* workspace, size_t workspace_bytes,
                                    hipEvent_t* events, int n_events, hipStream_t stream) {
  return sana::forward(q, k, v, out, B, N, H, d, eps, dtype, SANA_VARIANT_SPLIT, workspace,
                       workspace_bytes, events, n_events, nullptr, stream, fmap);
}

sana_status_t sana_linattn_fwd_strided(const void* q, const void* k, const void* v, int64_t ld,
                                       void* out, int64_t B, int64_t N, int64_t H, int64_t d,
                                       float eps, sana_dtype_t dtype, sana_fmap_t fmap, void* workspace,
                                       size_t workspace_bytes, hipEvent_t* events, int n_events,
                                       hipStream_t stream) {
  if (ld < 1) return SANA_ERR_INVALID_ARG;
  return sana::forward(q, k, v, out, B, N, H, d, eps, dtype, SANA_VARIANT_SPLIT, workspace,
                       workspace_bytes, events, n_events, nullptr, stream, fmap, ld);
}

sana_status_t sana_linattn_fwd(const void* q, const void* k, const void* v, void* out, int64_t B,
                               int64_t N, int64_t H, int64_t d, float eps, sana_dtype_t dtype,
                               void* workspace, size_t workspace_bytes, hipStream_t stream) {
  return sana_linattn_fwd_variant(q, k, v, out, B, N, H, d, eps, dtype, SANA_VARIANT_AUTO,
                                  workspace, workspace_bytes, stream);
}

sana_status_t sana_linattn_kv_state(const void* k, const void* v, float* state, int64_t B,
                                    int64_t N, int64_t H, int64_t d, sana_dtype_t dtype, void* workspace,
                                    size_t workspace_bytes, hipStream_t stream) {
  return sana_linattn_kv_state_fmap(k, v, state, B, N, H, d, dtype, SANA_FMAP_RELU, workspace,
                                    workspace_bytes, stream);
}

sana_status_t sana_linattn_kv_state_fmap(const void* k, const void* v, float* state, int64_t B,
                                         int64_t N, int64_t H, int64_t d, sana_dtype_t dtype,
                                         sana_fmap_t fmap, void* workspace,
                                         size_t workspace_bytes, hipStream_t stream) {
  size_t tb = 0;
  sana_status_t s = sana::check_shape(B, N, H, d, dtype, &tb);
  if (s != SANA_OK) return s;
  if (!sana::valid_fmap(fmap)) return SANA_ERR_UNSUPPORTED;
  if (!k || !v || !state) return SANA_ERR_INVALID_ARG;
  if (sana::misaligned(k) || sana::misaligned(v) || sana::misaligned(state))
    return SANA_ERR_ALIGNMENT;
  const Plan p = sana::make_plan(B, N, H);
  if ((s = sana::check_workspace(p, workspace, workspace_bytes)) != SANA_OK) return s;
  const size_t sb = static_cast<size_t>(B * H) * sana::kStateFloats * 4;
  if (sana::overlaps(state, sb, k, tb) || sana::overlaps(state, sb, v, tb) ||
      sana::overlaps(state, sb, workspace, p.workspace_bytes) ||
      sana::overlaps(workspace, p.workspace_bytes, k, tb) ||
      sana::overlaps(workspace, p.workspace_bytes, v, tb))
    return SANA_ERR_INVALID_ARG;
  (void)hipGetLastError();
  Plan fp = p;
  sana::fit_plan_to_device(fp, dtype);
  const sana::WorkspaceParts w = sana::split_workspace(fp, workspace);
  return sana::to_status(sana::launch_reduce(fp, dtype, true, k, v, w.partials, state, w.ctl,
                                             sana::next_epoch(), stream, fmap));
}

sana_status_t sana_linattn_apply(const void* q, const float* state, void* out, int64_t B,
                                 int64_t N, int64_t H, int64_t d, float eps, sana_dtype_t dtype,
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

sana_status_t sana_linattn_bwd_workspace_size(int64_t B, int64_t N, int64_t H, int64_t d,
                                              sana_dtype_t dtype, size_t* bytes) {
  if (!bytes) return SANA_ERR_INVALID_ARG;
  *bytes = 0;
  const sana_status_t s = sana::check_shape(B, N, H, d, dtype, nullptr);
  if (s != SANA_OK) return s;
  if (dtype != SANA_DTYPE_BF16) return SANA_ERR_UNSUPPORTED;
  *bytes = sana::bwd_workspace_bytes(sana::make_plan(B, N, H));
  return SANA_OK;
}

sana_status_t sana_linattn_bwd(const void* q, const void* k, const void* v, const void* dout,
                               void* dq, void* dk, void* dv, int64_t B, int64_t N, int64_t H,
                               int64_t d, float eps, sana_dtype_t dtype, void* workspace,
                               size_t workspace_bytes, hipStream_t stream) {
  return sana::backward(q, k, v, dout, dq, dk, dv, B, N, H, d, eps, dtype, workspace,
                        workspace_bytes, nullptr, 0, stream);
}

sana_status_t sana_linattn_bwd_profiled(const void* q, const void* k, const void* v,
                                        const void* dout, void* dq, void* dk, void* dv,
                                        int64_t B, int64_t N, int64_t H, int64_t d, float eps,
                                        sana_dtype_t dtype, void* workspace, size_t workspace_bytes,
                                        hipEvent_t* events, int n_events, hipStream_t stream) {
  if (!events) return SANA_ERR_INVALID_ARG;
  return sana::backward(q, k, v, dout, dq, dk, dv, B, N, H, d, eps, dtype, workspace,
                        workspace_bytes, events, n_events, stream);
}

sana_status_t sana_linattn_bwd_fmap(const void* q, const void* k, const void* v,
                                    const void* dout, void* dq, void* dk, void* dv, int64_t B,
                                    int64_t N, int64_t H, int64_t d, float eps,
                                    sana_dtype_t dtype, sana_fmap_t fmap, void* workspace,
                                    size_t workspace_bytes, hipEvent_t* events, int n_events,
                                    hipStream_t stream) {
  return sana::backward(q, k, v, dout, dq, dk, dv, B, N, H, d, eps, dtype, workspace,
                        workspace_bytes, events, n_events, stream, fmap);
}

sana_status_t sana_linattn_bwd_state(const void* q, const void* k, const void* v,
                                     const void* dout, const float* state, void* dq, void* dk,
                                     void* dv, int64_t B, int64_t N, int64_t H, int64_t d,
                                     float eps, sana_dtype_t dtype, sana_fmap_t fmap,
                                     void* workspace, size_t workspace_bytes, hipEvent_t* events,
                                     int n_events, hipStream_t stream) {
  return sana::backward(q, k, v, dout, dq, dk, dv, B, N, H, d, eps, dtype, workspace,
                        workspace_bytes, events, n_events, stream, fmap, state, true);
}

sana_status_t sana_linattn_block_causal_workspace_size(int64_t B, int64_t N, int64_t H,
                                                      int64_t d, int64_t block, sana_dtype_t dtype,
                                                      size_t* bytes) {
  if (!bytes) return SANA_ERR_INVALID_ARG;
  *bytes = 0;
  return sana::block_causal_workspace(B, N, H, d, block, dtype, bytes);
}

sana_status_t sana_linattn_fwd_block_causal(const void* q, const void* k, const void* v,
                                            void* out, int64_t B, int64_t N, int64_t H,
                                            int64_t d, int64_t block, float eps, sana_dtype_t dtype,
                                            void* workspace, size_t workspace_bytes,
                                            hipStream_t stream) {
  return sana::block_causal_any(q, k, v, out, B, N, H, d, block, eps, dtype, workspace,
                                workspace_bytes, nullptr, 0, stream);
}

sana_status_t sana_linattn_fwd_block_causal_profiled(const void* q, const void* k, const void* v,
                                                     void* out, int64_t B, int64_t N, int64_t H,
                                                     int64_t d, int64_t block, float eps,
                                                     sana_dtype_t dtype, void* workspace,
                                                     size_t workspace_bytes, hipEvent_t* events,
                                                     int n_events, hipStream_t stream) {
  if (!events) return SANA_ERR_INVALID_ARG;
  return sana::block_causal_any(q, k, v, out, B, N, H, d, block, eps, dtype, workspace,
                                workspace_bytes, events, n_events, stream);
}

sana_status_t sana_linattn_causal_workspace_size(int64_t B, int64_t N, int64_t H, int64_t d,
                                                sana_dtype_t dtype, size_t* bytes) {
  if (!bytes) return SANA_ERR_INVALID_ARG;
  *bytes = 0;
  sana::CausalPlan cp;
  size_t tb = 0;
  const sana_status_t s = sana::plan_causal(B, N, H, d, dtype, &cp, &tb);
  if (s != SANA_OK) return s;
  *bytes = cp.parts_bytes;
  return SANA_OK;
}

sana_status_t sana_linattn_fwd_causal(const void* q, const void* k, const void* v, void* out,
                                      int64_t B, int64_t N, int64_t H, int64_t d, float eps,
                                      sana_dtype_t dtype, void* workspace,
                                      size_t workspace_bytes, hipEvent_t* events, int n_events,
                                      hipStream_t stream) {
  return sana::causal_forward(q, k, v, out, B, N, H, d, eps, dtype, workspace, workspace_bytes,
                              events, n_events, stream);
}

sana_status_t sana_linattn_qkv_workspace_size(int64_t B, int64_t N, int64_t C, int64_t H,
                                              int64_t d, size_t* bytes) {
  if (!bytes) return SANA_ERR_INVALID_ARG;
  *bytes = 0;
  sana::QkvPlan qp;
  const sana_status_t s = sana::plan_qkv(B, N, C, H, d, &qp);
  if (s != SANA_OK) return s;
  *bytes = qp.workspace_bytes;
  return SANA_OK;
}

sana_status_t sana_linattn_qkv_fwd(const void* x, const void* w_qkv, void* q, void* out, int64_t B,
                                   int64_t N, int64_t C, int64_t H, int64_t d, float eps,
                                   void* workspace, size_t workspace_bytes, hipEvent_t* events,
                                   int n_events, hipStream_t stream) {
  return sana::qkv_forward(x, w_qkv, q, out, B, N, C, H, d, eps, workspace, workspace_bytes,
                           events, n_events, stream);
}

const char* sana_linattn_strerror(sana_status_t status) {
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
