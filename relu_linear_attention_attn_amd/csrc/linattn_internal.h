// Internal interface between the C ABI (api.cpp) and the HIP kernels
// (linattn_kernels.hip). Not installed; the public header is
// include/sana_linattn.h.
#pragma once

#include <cstddef>
#include <cstdint>

#include <hip/hip_runtime_api.h>

#include "sana_linattn.h"

namespace sana {

constexpr int kHeadDim = 32;                          // d
constexpr int kStateCols = kHeadDim + 1;              // d + 1: KV columns, then ksum
constexpr int kStateFloats = kHeadDim * kStateCols;   // 1056 floats = 4224 bytes
constexpr int kTile = 16;                             // tokens per wave iteration
constexpr int kHeadsPerBlock = 2;                     // a head pair shares 128-byte lines (bf16)

// Work split of one call. The bf16 reduction runs a (head-pair unit, token
// chunk) grid when one round of it fills the device, else blocks over
// balanced ranges of the flattened (unit, tile) index; the fp32 reduction
// and both applies run (unit, token chunk) grids. The block and chunk counts
// depend on the device (CU count and kernel occupancy); the workspace is
// sized for the largest counts any device can pick.
struct Plan {
  int64_t B, N, H;
  int64_t ld;             // elements between consecutive tokens of q, k and v
                          // (H * d unless the forward is called strided)
  int64_t pairs;          // ceil(H / 2) head pairs per batch item
  int64_t units;          // B * pairs
  int64_t tiles;          // 16-token tiles per unit, ceil(N / 16)
  // bf16 reduction: blocks and tiles per block (ranges of the flattened index)
  int64_t red_blocks, red_q;
  // bf16 reduction on a (unit, chunk) grid instead: red_cb chunks of red_cq
  // tiles per unit, one partial slot per chunk (red_cb = 0: balanced ranges)
  int64_t red_cb, red_cq;
  int64_t slots;          // partial slots per unit the workspace holds
  // token chunks (fp32 reduction; apply of both dtypes)
  int64_t red_chunk;      // tokens per reduction chunk (multiple of kTile)
  int64_t red_chunks;     // chunks used (<= red_chunks_max)
  int64_t red_chunks_max; // chunks the workspace is sized for
  int64_t app_chunk;      // tokens per apply chunk (multiple of kTile)
  int64_t app_chunks;
  // bf16 apply on balanced ranges instead: app_blocks blocks of app_q tiles
  // of the flattened (unit, tile) index (app_q = 0: the (unit, chunk) grid)
  int64_t app_q, app_blocks;
  int64_t bkv_chunk;      // backward k/v pass (bf16): tokens per chunk, chunks per unit
  int64_t bkv_chunks;
  size_t partial_bytes;   // workspace bytes for partials (either dtype)
  size_t bf16_partial_bytes;  // of which the bf16 partials need
  size_t state_bytes;     // workspace bytes for the combined state
  size_t ctl_bytes;       // workspace bytes for the per-unit control words
  size_t workspace_bytes; // total
};

// The slot rule of the bf16 reduction's partials: -chunks per unit on a
// (unit, chunk) grid, else the tiles per balanced range (each unit's slot
// count follows from it, see the kernels' slot_count).
inline int64_t red_rule(const Plan& p) { return p.red_cb > 0 ? -p.red_cb : p.red_q; }

// Supplies a workspace (device pointer and bytes) to the forward pass; asked
// only after every host check of the call has passed.
typedef hipError_t (*WorkspaceSource)(void** workspace, size_t* bytes);

// sana_linattn_fwd with its workspace taken from `ws_source` (api.cpp).
sana_status_t forward_from_source(const void* q, const void* k, const void* v, void* out,
                                  int64_t B, int64_t N, int64_t H, int64_t d, float eps,
                                  int dtype, WorkspaceSource ws_source, hipStream_t stream);

// Device-independent part of the plan: sizes and the workspace layout.
Plan make_plan(int64_t B, int64_t N, int64_t H);
// Fills the chunk counts for the current device (makes HIP queries once per device).
void fit_plan_to_device(Plan& p, int dtype);

enum class KernelKind { kReduce, kApply, kBwdQ, kBwdKV };
int occupancy_blocks_per_cu(KernelKind kind, int dtype);
int block_waves(KernelKind kind, int dtype);  // waves per block

// Launchers. They enqueue on `stream` and return the launch status.
// dtype: 0 = fp32, 1 = bf16 (sana_dtype_t). The reduction writes per-block
// partials; with fold (always for fp32) the last block of each head pair
// also folds them into `state`, without (bf16) the partials are the result
// and launch_apply_partials sums them where it needs them.
// fmap is the feature map (sana_fmap_t).
// keep_k (bf16 partials only): k is read with ordinary loads, which leave
// much of it in the Infinity Cache for a later pass that reads it again (the
// backward's k/v pass); otherwise k and v with streaming loads.
hipError_t launch_reduce(const Plan& p, int dtype, bool fold, const void* k, const void* v,
                         float* partials, float* state, unsigned long long* ctl,
                         unsigned long long epoch, hipStream_t stream, int fmap = 0,
                         bool keep_k = false);
// Apply from a folded [B][H][d][d+1] state.
hipError_t launch_apply(const Plan& p, int dtype, const void* q, const float* state,
                        void* out, float eps, hipStream_t stream, int fmap = 0);
// bf16 apply from the partials of launch_reduce(fold = false) with the same plan.
hipError_t launch_apply_partials(const Plan& p, const void* q, const float* partials, void* out,
                                 float eps, hipStream_t stream, int fmap = 0);
// bf16 apply from `count` partial slots per unit laid out [units][count][2][d][d+1].
hipError_t launch_apply_slots(const Plan& p, const void* q, const float* partials, int64_t count,
                              void* out, float eps, hipStream_t stream);
// QKV projection with the state in its epilogue (qkv_kernels.hip): writes q
// [B][N][H][d] bf16 and one partial state per (batch item, head pair,
// 256-token tile), [B][pairs][qkv_m_tiles(N)][2][d][d+1] fp32. GM: M tiles
// per group of the block order.
int64_t qkv_m_tiles(int64_t N);
int64_t qkv_grid_blocks(int64_t B, int64_t N, int64_t H);
hipError_t launch_qkv_state(const void* x, const void* w, void* q, float* partials, int64_t B,
                            int64_t N, int64_t C, int64_t H, int64_t GM, hipStream_t stream);
// Backward (bf16). bwd_q runs on the state reduction's grid: it sums the
// partials of launch_reduce(fold = false) for the state (slots by
// red_rule), writes dq and writes [dS | dz] partials in the same slots (same
// rule); bwd_kv sums those and writes dk and dv.
// fmap: the feature map (sana_fmap_t values) whose backward the passes take
// state: a folded fp32 [B][H][d][d+1] forward state to take instead of the
// partials fwd_parts (NULL: the partials).
hipError_t launch_bwd_q(const Plan& p, const void* q, const void* g, void* dq,
                        const float* fwd_parts, const float* state, float* grad_parts, float eps,
                        hipStream_t stream, int fmap);
hipError_t launch_bwd_kv(const Plan& p, const void* k, const void* v, void* dk, void* dv,
                         const float* grad_parts, hipStream_t stream, int fmap);
// Block-causal attention: p's batch items are the F blocks of each of the
// p.B / F original batch items. Inclusive prefix sums over the blocks of the
// reduction's result (bf16: its partials, launch_reduce(fold = false);
// fp32: its folded state) into prefix, a [p.B][H][d][d+1] state for
// launch_apply.
// Token-causal attention (bf16): chunk states, their exclusive prefix,
// then the causal apply. One wave per (unit, chunk of W consecutive tiles);
// W chosen so the units' chunks make one round of about kCausalWaves waves.
// The same plan serves block-causal attention with short bf16 blocks: blocks
// of 2^lg <= 16 tokens on the causal apply, blocks of m whole tiles on the
// block-wise apply (W then a multiple of m).
constexpr int64_t kCausalWaves = 2048;      // 8 waves on each of 256 CUs
constexpr int64_t kMaxCausalChunks = 1024;  // per unit
struct CausalPlan {
  int64_t B, N, H, pairs, units, tiles, chunks, W;
  int lg;              // blocks of 2^lg tokens (0: token-causal; at most 4)
  int64_t m;           // > 1: blocks of m whole tiles (the block-wise apply); W a multiple
  size_t parts_bytes;  // [units][chunks][2][d][d+1] fp32
};
hipError_t launch_causal_states(const CausalPlan& cp, const void* k, const void* v, float* parts,
                                hipStream_t stream);
hipError_t launch_causal_scan(const CausalPlan& cp, float* parts, hipStream_t stream);
hipError_t launch_causal_block_apply(const CausalPlan& cp, const void* q, const void* k,
                                     const void* v, void* out, const float* parts, float eps,
                                     hipStream_t stream);
hipError_t launch_causal_apply(const CausalPlan& cp, const void* q, const void* k, const void* v,
                               void* out, const float* parts, float eps, hipStream_t stream);
hipError_t launch_scan_blocks(const Plan& p, int dtype, int64_t F, const float* partials,
                              const float* state, float* prefix, hipStream_t stream);
int64_t scan_grid_threads(int64_t B, int64_t pairs);  // work-items of that launch
// cus: the device's CU count, which picks the bf16 block shape (waves per
// block and tiles in flight per wave) from the head-pair units per CU.
hipError_t launch_fused(const Plan& p, int dtype, int64_t cus, const void* q, const void* k,
                        const void* v, void* out, float eps, hipStream_t stream);

}  // namespace sana
