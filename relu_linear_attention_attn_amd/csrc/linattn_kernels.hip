// HIP kernels (gfx950) for the ReLU linear self-attention forward pass.
//
// Per (b, h): state = phi(K)^T [V | 1] (d x (d+1), fp32), then
// out_i = phi(q_i) state[:, :d] / (phi(q_i) . state[:, d] + eps).
// Sources: Sana course notes, "Linear Attention 的原理" (phi = ReLU, the d x d
// state, A = phi(Q) KV); Linear-DiT 4K blog, "核心架构" (the normaliser
// phi(Q) phi(K)^T 1); Sana paper review, section 2.2 "선형 어텐션 블럭" (shared
// terms computed once per head and reused by every query). The review's
// "Triton을 통한 학습/추론 가속화" names the element-wise work to keep inside
// the contractions (activation, precision conversion, padding, division):
// here ReLU runs on packed bf16 in registers, the [V | 1] column is carried
// alongside (ksum summed from the same registers in the reduction, a third
// MFMA tile in the apply), the division is one reciprocal per token, and the
// bf16 rounding happens on the store.
//
// Tensors are [B][N][H][d], d = 32. One wave owns one head over a run of
// 16-token tiles; a block holds a head pair (2 x 64 bytes = one 128-byte line
// per token in bf16) times S token sub-streams.
//
// bf16 path (the hot path), both halves on the matrix cores:
//   reduce: state += phi(K_tile)^T V_tile with v_mfma_f32_32x32x16_bf16
//           (rows = k channel, cols = v channel, contraction over 16 tokens).
//           MFMA wants 8 consecutive tokens of one channel per lane, while
//           memory holds 8 consecutive channels of one token, so each tile
//           is staged through the wave's own LDS slot and gathered back
//           transposed. ksum is summed on the VALU from the same gathered
//           phi(k) values, each widened exactly from bf16.
//   apply:  out^T = KV^T phi(Q_tile)^T with v_mfma_f32_16x16x32_bf16, K = d
//           in one instruction. The fp32 state is split into bf16 hi + lo
//           parts (x = hi + lo to ~2^-17 relative), so the products keep
//           near-fp32 accuracy; phi(q) is exact in bf16. The output rows of
//           the two 16-row MFMA tiles are permuted so each lane ends up with
//           8 consecutive output channels of one token: one 16-byte store.
//           The denominator comes from a third tile whose A rows all equal
//           ksum, so it lands in the same lane and register as its numerator.
// fp32 path: the same two halves on fp32 MFMA (v_mfma_f32_32x32x2f32: exact
// fp32 products and fp32 sums, for the fp32 contract) over 32-token tiles of
// one head.

#include <hip/hip_runtime.h>

#include <type_traits>

#include "linattn_internal.h"

namespace sana {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef short s16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));

constexpr int kWave = 64;
constexpr int kD = kHeadDim;      // 32
constexpr int kSC = kStateCols;   // 33
constexpr int kSF = kStateFloats; // 1056

__device__ __forceinline__ int lane_id() { return threadIdx.x & (kWave - 1); }

// Orders this wave's LDS accesses: LDS requests of one wave are served in
// issue order, so only the compiler must be kept from moving them across.
__device__ __forceinline__ void wave_lds_order() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

__device__ __forceinline__ void st16(void* p, u32x4 x) { *reinterpret_cast<u32x4*>(p) = x; }

// Streaming (nontemporal) accesses for data touched exactly once per call:
// the token tensors every kernel reads (Q, K, V, dOut) and writes (Out, dQ,
// dK, dV). They keep the single-use lines from displacing others in L2 and
// the Infinity Cache, and let output lines go to HBM while the kernel runs
// instead of being evicted, dirty, during the next call's reads.
// An ordinary (temporal) load: the line is kept in the caches on the way,
// the Infinity Cache included, for a kernel that reads it again soon.
__device__ __forceinline__ u32x4 ld16_keep(const void* p) {
  return *reinterpret_cast<const u32x4*>(p);
}
__device__ __forceinline__ u32x4 ld16_stream(const void* p) {
  return __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
}
__device__ __forceinline__ void st16_stream(void* p, u32x4 x) {
  __builtin_nontemporal_store(x, reinterpret_cast<u32x4*>(p));
}

// ReLU on 8 packed bf16: a bf16 compares like its int16 bit pattern against
// +0 (negative values and -0 have the sign bit set), so max(x, 0) as signed
// 16-bit integers is the float ReLU.
__device__ __forceinline__ u32x4 relu_bf16x8(u32x4 x) {
  s16x8 s = __builtin_bit_cast(s16x8, x);
  s = __builtin_elementwise_max(s, (s16x8)0);
  return __builtin_bit_cast(u32x4, s);
}

// 8 packed bf16 -> fp32 (exact: a bf16 is the top half of a binary32).
__device__ __forceinline__ void widen_bf16x8(u32x4 w, float (&x)[8]) {
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    x[2 * e] = __builtin_bit_cast(float, w[e] << 16);
    x[2 * e + 1] = __builtin_bit_cast(float, w[e] & 0xFFFF0000u);
  }
}

typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef short s16x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

// Two floats to two bf16 (round to nearest even), as one packed conversion.
__device__ __forceinline__ unsigned int cvt_pk_bf16(float a, float b) {
  return __builtin_bit_cast(unsigned int, __builtin_convertvector((f32x2){a, b}, bf16x2));
}

// The ReLU gate on a packed bf16 pair: v kept in each half where the same
// half of relu (max(x, 0) of x's bits as signed 16-bit values) is nonzero,
// i.e. x > 0, and zeroed elsewhere. relu's halves are 0 or 0x0001..0x7FFF, so
// adding 0x7FFF to each (no carry crosses: at most 0xFFFE) sets a half's top
// bit exactly where x > 0, and an arithmetic shift spreads it over the half.
__device__ __forceinline__ unsigned int relu_gate_pk(unsigned int v, unsigned int relu) {
  const s16x2 top = __builtin_bit_cast(s16x2, relu + 0x7FFF7FFFu);
  return v & __builtin_bit_cast(unsigned int, top >> 15);
}

// x = hi + lo with hi = bf16(x) and lo = bf16(x - hi) (x to ~2^-17 relative),
// a pair at a time: one packed conversion each for hi and lo, hi widened back
// exactly (a bf16 is the top half of a binary32).
__device__ __forceinline__ void split_bf16x8(const float (&x)[8], bf16x8& hi, bf16x8& lo) {
  u32x4 h, w;
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    h[e] = cvt_pk_bf16(x[2 * e], x[2 * e + 1]);
    const float h0 = __builtin_bit_cast(float, h[e] << 16);
    const float h1 = __builtin_bit_cast(float, h[e] & 0xFFFF0000u);
    w[e] = cvt_pk_bf16(x[2 * e] - h0, x[2 * e + 1] - h1);
  }
  hi = __builtin_bit_cast(bf16x8, h);
  lo = __builtin_bit_cast(bf16x8, w);
}

// Feature maps phi, element by element in fp32 (the values of sana_fmap_t):
// ReLU; ELU + 1 with alpha = 1 (x + 1 above 0, exp(x) at or below); cos.
// ReLU of a bf16 is a bf16, and the bf16 kernels keep their packed ReLU
// path for it; the other maps are not exact in bf16, so the bf16 kernels
// split phi into bf16 hi + lo parts for the MFMAs.
constexpr int kFmapRelu = 0, kFmapElu1 = 1, kFmapCos = 2;
template <int Fm>
__device__ __forceinline__ float fmap_f32(float x) {
  if (Fm == kFmapElu1) return x > 0.0f ? x + 1.0f : expf(x);
  if (Fm == kFmapCos) return cosf(x);
  return fmaxf(x, 0.0f);
}
// The same maps from the hardware's transcendental instructions, for the
// bf16 kernels, whose phi feeds bf16 hi + lo MFMA operands: exp(x) as
// 2^(x log2 e) (v_exp_f32) and cos(x) as v_cos_f32 of the fraction of
// x / (2 pi) in revolutions. Measured against double-precision exp and cos:
// cos within 4e-7 absolute for |x| < 4 (3e-6 for |x| < 40, the argument
// scaling's rounding), exp within 2e-6 relative on (-40, 0] - far below the
// bf16 output rounding (2^-9). The library routines cost several times as
// many instructions and made both kernels compute-bound (ELU + 1 forward at
// 2 x 16384 x 70: 164 -> 133 us; cos: 195 -> 129 us).
template <int Fm>
__device__ __forceinline__ float fmap_hw(float x) {
  constexpr float kLog2e = 1.4426950408889634f;
  constexpr float kInv2Pi = 0.15915494309189535f;
  if (Fm == kFmapElu1) return x > 0.0f ? x + 1.0f : __builtin_amdgcn_exp2f(x * kLog2e);
  if (Fm == kFmapCos) return __builtin_amdgcn_cosf(__builtin_amdgcn_fractf(x * kInv2Pi));
  return fmaxf(x, 0.0f);
}
// phi(x), as fmap_hw gives it, and phi'(x) from the same instructions, for
// the backward pass: ELU + 1 has 1 above 0 and exp(x) at or below it
// (continuous at 0; that exp(x) is phi there too), cos has -sin(x) (v_sin_f32
// of the same fraction of revolutions); ReLU's is taken as 0 at 0.
template <int Fm>
__device__ __forceinline__ void fmap_dfmap_hw(float x, float& phi, float& dphi) {
  constexpr float kLog2e = 1.4426950408889634f;
  constexpr float kInv2Pi = 0.15915494309189535f;
  if (Fm == kFmapElu1) {
    const float e = __builtin_amdgcn_exp2f(x * kLog2e);
    phi = x > 0.0f ? x + 1.0f : e;
    dphi = x > 0.0f ? 1.0f : e;
  } else if (Fm == kFmapCos) {
    const float r = __builtin_amdgcn_fractf(x * kInv2Pi);
    phi = __builtin_amdgcn_cosf(r);
    dphi = -__builtin_amdgcn_sinf(r);
  } else {
    phi = fmaxf(x, 0.0f);
    dphi = x > 0.0f ? 1.0f : 0.0f;
  }
}

// -------------------------------------------------- line tiles in LDS
//
// A wave owns a head pair (h, h+1): per token that is one 128-byte line of
// the [B][N][H][d] bf16 tensor (two 64-byte head rows). Every global load and
// store moves whole lines: lane l handles 16-byte piece l%8 of tokens l/8 and
// 8 + l/8 of a 16-token tile, so one instruction covers 8 full lines (whole
// lines are what keeps the HBM write path at full rate). The tile is staged
// in the wave's own LDS slot as 16 rows of 128 bytes; piece j of token t sits
// in slot j ^ ((t >> 1) & 7) of its row. That swizzle makes the column reads
// of the MFMA layouts (16 tokens, one piece) and the line reads both free of
// bank conflicts.
constexpr int kLineBytes = 128;
constexpr int kTileBytes = kTile * kLineBytes;  // 2 KB

__device__ __forceinline__ int tile_off(int t, int j) {
  return (t << 7) + ((j ^ ((t >> 1) & 7)) << 4);
}

typedef short s16x4 __attribute__((ext_vector_type(4)));

// The 32x32x16 MFMA operand of head hh from a staged tile: lane l gets
// channel l % 32 of the 8 tokens 8 (l / 32) .. + 7 (packed bf16, token
// order), read with two gfx950 LDS transpose loads. In each 16-lane group,
// ds_read_b64_tr_b16 hands lane l element l % 4 of the 64-bit rows read by
// lanes 4 k + l / 4, k = 0..3 (checked on the device); so lane r of the
// group reads token t + r / 4, channels c + 4 (r % 4) .. + 3, and lane l then
// holds channel c + l % 16 of tokens t .. t + 3. The same values as sixteen
// 16-bit reads, in a quarter of the instructions and without packing.
__device__ __forceinline__ s16x8 gather_tokens8(const unsigned char* tile, int hh) {
  typedef __attribute__((address_space(3))) s16x4 lds_s16x4;
  const int l = lane_id();
  const int grp = l >> 4, r = l & 15;
  const int c = 16 * (grp & 1) + 4 * (r & 3);   // first of the row's 4 channels
  const int t = 8 * (grp >> 1) + (r >> 2);       // the row's token, first half
  const int j = hh * 4 + (c >> 3);
  const s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
      (lds_s16x4*)(tile + tile_off(t, j) + 2 * (c & 7)));
  const s16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
      (lds_s16x4*)(tile + tile_off(t + 4, j) + 2 * (c & 7)));
  return (s16x8){lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
}

template <bool Coherent>
__device__ __forceinline__ void put(float* p, float x) {
  if (Coherent) {
    __hip_atomic_store(p, x, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  } else {
    *p = x;
  }
}

// ------------------------------------------------------------ bf16 reduce

// Accumulates phi(K)^T V (into acc, MFMA layout) and phi(K)^T 1 (into ks:
// lane l sums channel l%32 over the tokens it gathers) for the head pair over
// the tiles sub, sub + S, ... of the token range [n_lo, n_hi). `base` is the
// element offset of (b, n = 0, h, c = 0) for the pair's first head, `row` the
// element stride between tokens. `two` says whether the pair's second head
// exists (H odd leaves the last pair with one head: its lanes then read the
// first head's half-line again, which stays inside the tensor, and the second
// head's sums are discarded). KeepK / KeepV: that tensor is read with
// ordinary loads, which leave it in the caches (the Infinity Cache included)
// for a later pass; otherwise with streaming loads.
template <int U, int Fm = kFmapRelu, bool KeepK = false, bool KeepV = false>
__device__ __forceinline__ void reduce_pair_wave(const unsigned short* __restrict__ K,
                                                 const unsigned short* __restrict__ V,
                                                 int64_t row, int64_t base, int64_t n_lo,
                                                 int64_t n_hi, int sub, int S, bool two,
                                                 unsigned char* slot, f32x16 (&acc)[2],
                                                 float (&ks)[2]) {
  const int l = lane_id();
  const int t0 = l >> 3;
  const int j = l & 7;
  const int jl = two ? j : (j & 3);
  const int rt = (l >> 5) * 8;     // first of the 8 tokens this lane gathers
  const int64_t tiles = (n_hi - n_lo + kTile - 1) / kTile;
  const int64_t mine = tiles > sub ? (tiles - sub + S - 1) / S : 0;

  // Loads are never predicated: a token outside the range (ragged tail, or a
  // tile past the end) reads row n_lo instead, which is always inside the
  // tensor, and its k is zeroed when staged (ReLU(0) = 0 drops the token from
  // both KV and ksum; for the other maps phi itself is zeroed past the
  // tile's `valid` tokens). Unconditional loads keep U tiles in flight.
  u32x4 kb[U][2], vb[U][2];
  auto issue = [&](int64_t i, u32x4 (&kd)[2], u32x4 (&vd)[2]) {
    const int64_t n0 = n_lo + (sub + i * S) * kTile + t0;
#pragma unroll
    for (int h2 = 0; h2 < 2; ++h2) {
      const int64_t n = n0 + 8 * h2;
      const int64_t off = base + (n < n_hi ? n : n_lo) * row + 8 * jl;
      kd[h2] = KeepK ? ld16_keep(K + off) : ld16_stream(K + off);
      vd[h2] = KeepV ? ld16_keep(V + off) : ld16_stream(V + off);
    }
  };
#pragma unroll
  for (int u = 0; u < U; ++u) issue(u, kb[u], vb[u]);

  auto stage = [&](int64_t i, const u32x4 (&kin)[2], const u32x4 (&vin)[2]) {
    const int64_t n0 = n_lo + (sub + i * S) * kTile + t0;
#pragma unroll
    for (int h2 = 0; h2 < 2; ++h2) {
      const int o = tile_off(t0 + 8 * h2, j);
      *reinterpret_cast<u32x4*>(slot + o) = n0 + 8 * h2 < n_hi ? kin[h2] : (u32x4)0;
      *reinterpret_cast<u32x4*>(slot + kTileBytes + o) = vin[h2];
    }
  };
  auto valid_in = [&](int64_t i) {
    const int64_t left = n_hi - (n_lo + (sub + i * S) * kTile);
    return static_cast<int>(left < kTile ? left : kTile);
  };
  auto consume = [&](int valid) {
    wave_lds_order();
    s16x8 a[2], bv[2];
#pragma unroll
    for (int hh = 0; hh < 2; ++hh) {
      a[hh] = gather_tokens8(slot, hh);
      bv[hh] = gather_tokens8(slot + kTileBytes, hh);
    }
    wave_lds_order();
    if (Fm == kFmapRelu) {
#pragma unroll
      for (int hh = 0; hh < 2; ++hh) {
        const s16x8 pk = __builtin_elementwise_max(a[hh], (s16x8)0);   // phi(k), packed
        acc[hh] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, pk),
                                                          __builtin_bit_cast(bf16x8, bv[hh]),
                                                          acc[hh], 0, 0, 0);
        // ksum: widen each bf16 exactly (it is the top half of a binary32) and add
        const u32x4 w = __builtin_bit_cast(u32x4, pk);
        float sum = 0.0f;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          sum += __builtin_bit_cast(float, w[e] << 16);
          sum += __builtin_bit_cast(float, w[e] & 0xFFFF0000u);
        }
        ks[hh] += sum;
      }
    } else {
      // phi in fp32, zero past the tile's valid tokens, split hi + lo
      // against the exact v (two MFMAs); ksum from the fp32 values
#pragma unroll
      for (int hh = 0; hh < 2; ++hh) {
        float x[8];
        widen_bf16x8(__builtin_bit_cast(u32x4, a[hh]), x);
        float sum = 0.0f;
#pragma unroll
        for (int s = 0; s < 8; ++s) {
          x[s] = rt + s < valid ? fmap_hw<Fm>(x[s]) : 0.0f;
          sum += x[s];
        }
        bf16x8 hi, lo;
        split_bf16x8(x, hi, lo);
        const bf16x8 vb8 = __builtin_bit_cast(bf16x8, bv[hh]);
        acc[hh] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(hi, vb8, acc[hh], 0, 0, 0);
        acc[hh] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(lo, vb8, acc[hh], 0, 0, 0);
        ks[hh] += sum;
      }
    }
  };
  // Main loop: whole groups of U tiles and no branches inside, so the load
  // counter stays exact and U tiles stay in flight.
  int64_t i0 = 0;
  for (; i0 + U <= mine; i0 += U) {
#pragma unroll
    for (int u = 0; u < U; ++u) {
      stage(i0 + u, kb[u], vb[u]);
      // refill kb[u], vb[u] only after their last use, so they keep their registers
      __builtin_amdgcn_sched_barrier(0);
      issue(i0 + u + U, kb[u], vb[u]);
      consume(valid_in(i0 + u));
    }
  }
#pragma unroll
  for (int u = 0; u < U; ++u) {
    if (i0 + u < mine) {
      stage(i0 + u, kb[u], vb[u]);
      consume(valid_in(i0 + u));
    }
  }
}

// Where a launch must leave one folded state (the fp32 reduction, and the
// bf16 one behind sana_linattn_kv_state), the partials of a head pair are
// folded into it by the last block to finish that pair, in ascending chunk
// order, so the result does not depend on which block finishes last. The
// hand-off between blocks (which may sit on different XCDs, each with its
// own L2) is a release/acquire pair at agent scope on the pair's control
// word:
//   * partials are written with agent-scope (device-coherent) stores, and
//     each wave waits until its stores have completed before the block
//     barrier, so every store of the block precedes thread 0's update;
//   * thread 0 counts the block in with a compare-and-swap that is a release
//     (the block's partials become visible device-wide before the new count
//     can be seen) and an acquire (if it is the last block, the other
//     blocks' partials, released before their counts, are visible to it);
//   * the last block reads the partials back with agent-scope loads after
//     the block barrier that follows thread 0's acquire.
// The control word holds (call epoch << 16 | finished blocks). A word left by
// an earlier call, or garbage, carries another epoch and restarts the count,
// so the workspace needs no clearing between calls. The last block also sets
// the word back to 0 (a tag no call carries) once every block has counted
// in: a launch replayed with the same epoch (a captured HIP graph) then
// starts its count afresh too.
__device__ __forceinline__ float load_coherent(const float* p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

__device__ __forceinline__ bool arrive_last(unsigned long long* ctl, unsigned long long epoch,
                                            int64_t nchunks) {
  __shared__ int last;
  // wait until this wave's partial stores have completed
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  __syncthreads();
  if (threadIdx.x == 0) {
    unsigned long long cur = __hip_atomic_load(ctl, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    unsigned long long nxt;
    while (true) {
      nxt = (cur >> 16) == epoch ? cur + 1 : ((epoch << 16) | 1ull);
      if (__hip_atomic_compare_exchange_strong(ctl, &cur, nxt, __ATOMIC_ACQ_REL,
                                               __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT))
        break;
    }
    last = static_cast<int64_t>(nxt & 0xFFFFull) == nchunks;
    // every block of the pair has counted in: nothing else touches the word
    if (last) __hip_atomic_store(ctl, 0ull, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
  __syncthreads();
  return last != 0;
}

// dst[e] = sum_{p < P} src[p * stride + e] for e < n, in ascending p. All
// loads of a batch are issued before any is added, so the fold costs about
// one memory round trip per 16 partials.
__device__ __forceinline__ void fold_partials(const float* __restrict__ src, int64_t stride,
                                             float* __restrict__ dst, int n, int64_t P) {
  constexpr int kBatch = 16;
  for (int e = threadIdx.x; e < n; e += blockDim.x) {
    float acc = 0.0f;
    for (int64_t p0 = 0; p0 < P; p0 += kBatch) {
      float x[kBatch];
#pragma unroll
      for (int u = 0; u < kBatch; ++u)
        x[u] = p0 + u < P ? load_coherent(src + (p0 + u) * stride + e) : 0.0f;
#pragma unroll
      for (int u = 0; u < kBatch; ++u)
        if (p0 + u < P) acc = (p0 + u == 0) ? x[u] : acc + x[u];
    }
    dst[e] = acc;
  }
}

// ------------------------------------------------------------- bf16 apply

struct ApplyOperands {
  bf16x8 kv0_hi, kv0_lo, kv1_hi, kv1_lo, ks_hi, ks_lo;
};

// Builds the A operands of the three 16x16x32 MFMA tiles from a [d][d+1]
// fp32 state. A lane supplies row i = l%16 and contraction indices
// k = 8*(l/16) + s, s = 0..7 (the same k the lane reads from q). Tile t row i
// stands for output channel 8*(i/4) + 4t + i%4, so after the MFMA a lane
// holds output channels 8*(l/16) .. +7 of token l%16.
__device__ __forceinline__ ApplyOperands make_apply_operands(const float* st) {
  const int l = lane_id();
  const int g = l >> 4;
  const int i = l & 15;
  ApplyOperands o;
#pragma unroll
  for (int s = 0; s < 8; ++s) {
    const int c = 8 * g + s;
    const float x0 = st[c * kSC + 8 * (i >> 2) + (i & 3)];
    const float x1 = st[c * kSC + 8 * (i >> 2) + 4 + (i & 3)];
    const float xs = st[c * kSC + kD];
    const __bf16 h0 = (__bf16)x0, h1 = (__bf16)x1, hs = (__bf16)xs;
    o.kv0_hi[s] = h0;
    o.kv0_lo[s] = (__bf16)(x0 - (float)h0);
    o.kv1_hi[s] = h1;
    o.kv1_lo[s] = (__bf16)(x1 - (float)h1);
    o.ks_hi[s] = hs;
    o.ks_lo[s] = (__bf16)(xs - (float)hs);
  }
  return o;
}

// One head's 16-token output: phi(q) from the operand-layout piece, six
// MFMAs, one reciprocal per token, bf16 rounding. Returns the lane's 8
// output channels (one 16-byte piece) of token l%16.
// For maps other than ReLU, phi(q) is split into hi + lo too and three
// more MFMAs add the state's hi parts times phi(q)'s lo part.
template <int Fm = kFmapRelu>
__device__ __forceinline__ u32x4 apply_head(const ApplyOperands& op, u32x4 qpiece, float eps) {
  f32x4 a0, a1, ad;
  if (Fm == kFmapRelu) {
    const bf16x8 qv = __builtin_bit_cast(bf16x8, relu_bf16x8(qpiece));
    a0 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(op.kv0_hi, qv, (f32x4)0, 0, 0, 0);
    a0 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(op.kv0_lo, qv, a0, 0, 0, 0);
    a1 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(op.kv1_hi, qv, (f32x4)0, 0, 0, 0);
    a1 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(op.kv1_lo, qv, a1, 0, 0, 0);
    ad = __builtin_amdgcn_mfma_f32_16x16x32_bf16(op.ks_hi, qv, (f32x4)0, 0, 0, 0);
    ad = __builtin_amdgcn_mfma_f32_16x16x32_bf16(op.ks_lo, qv, ad, 0, 0, 0);
  } else {
    float x[8];
    widen_bf16x8(qpiece, x);
#pragma unroll
    for (int m = 0; m < 8; ++m) x[m] = fmap_hw<Fm>(x[m]);
    bf16x8 qh, ql;
    split_bf16x8(x, qh, ql);
    a0 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(op.kv0_hi, qh, (f32x4)0, 0, 0, 0);
    a0 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(op.kv0_lo, qh, a0, 0, 0, 0);
    a0 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(op.kv0_hi, ql, a0, 0, 0, 0);
    a1 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(op.kv1_hi, qh, (f32x4)0, 0, 0, 0);
    a1 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(op.kv1_lo, qh, a1, 0, 0, 0);
    a1 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(op.kv1_hi, ql, a1, 0, 0, 0);
    ad = __builtin_amdgcn_mfma_f32_16x16x32_bf16(op.ks_hi, qh, (f32x4)0, 0, 0, 0);
    ad = __builtin_amdgcn_mfma_f32_16x16x32_bf16(op.ks_lo, qh, ad, 0, 0, 0);
    ad = __builtin_amdgcn_mfma_f32_16x16x32_bf16(op.ks_hi, ql, ad, 0, 0, 0);
  }
  const float rinv = 1.0f / (ad[0] + eps);
  bf16x8 o;
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    o[r] = (__bf16)(a0[r] * rinv);
    o[4 + r] = (__bf16)(a1[r] * rinv);
  }
  return __builtin_bit_cast(u32x4, o);
}

// Applies the pair's two heads to the tiles sub, sub + S, ... of [n_lo, n_hi).
// `two` as for reduce_pair_wave: with one head, the second half-line is read
// from the first head (inside the tensor), computed and never stored.
// pre_ops() runs first and returns what make_ops(op, pre) needs loaded
// ahead (the first state slots); make_ops fills the two heads' operands
// after the first U tiles' loads are issued, so whatever it waits for (the
// state's loads, a block barrier: every wave of the block calls it) overlaps
// those loads, and the state's loads, issued before them, do not wait
// behind them.
// row / base locate q as in reduce_pair_wave; orow / obase locate the output.
template <int U, int Fm = kFmapRelu, class PreOps, class MakeOps>
__device__ __forceinline__ void apply_pair_wave(const unsigned short* __restrict__ Q,
                                                unsigned short* __restrict__ Out,
                                                PreOps&& pre_ops, MakeOps&& make_ops, float eps,
                                                int64_t row, int64_t base, int64_t orow,
                                                int64_t obase, int64_t n_lo, int64_t n_hi,
                                                int sub, int S, bool two,
                                                unsigned char* slot) {
  const int l = lane_id();
  const int t0 = l >> 3;
  const int j = l & 7;
  const int jl = two ? j : (j & 3);
  const int g = l >> 4;
  const int col = l & 15;
  const int64_t tiles = (n_hi - n_lo + kTile - 1) / kTile;
  const int64_t mine = tiles > sub ? (tiles - sub + S - 1) / S : 0;

  // Unpredicated loads (see reduce_pair_wave): an out-of-range token reads
  // row n_lo and its result is simply not stored.
  u32x4 qb[U][2];
  auto issue = [&](int64_t i, u32x4 (&qd)[2]) {
    const int64_t n0 = n_lo + (sub + i * S) * kTile + t0;
#pragma unroll
    for (int h2 = 0; h2 < 2; ++h2) {
      const int64_t n = n0 + 8 * h2;
      qd[h2] = ld16_stream(Q + base + (n < n_hi ? n : n_lo) * row + 8 * jl);
    }
  };
  const auto pre = pre_ops();
#pragma unroll
  for (int u = 0; u < U; ++u) issue(u, qb[u]);
  ApplyOperands op[2];
  make_ops(op, pre);

  // stage the tile's lines, compute both heads in place in the tile, and read
  // the output lines back; `full` says the whole tile is inside the range
  auto compute = [&](const u32x4 (&qin)[2]) {
#pragma unroll
    for (int h2 = 0; h2 < 2; ++h2)
      *reinterpret_cast<u32x4*>(slot + tile_off(t0 + 8 * h2, j)) = qin[h2];
    wave_lds_order();
    u32x4 qp[2];
#pragma unroll
    for (int hh = 0; hh < 2; ++hh)
      qp[hh] = *reinterpret_cast<const u32x4*>(slot + tile_off(col, hh * 4 + g));
    wave_lds_order();
#pragma unroll
    for (int hh = 0; hh < 2; ++hh)
      *reinterpret_cast<u32x4*>(slot + tile_off(col, hh * 4 + g)) =
          apply_head<Fm>(op[hh], qp[hh], eps);
    wave_lds_order();
  };
  auto out_line = [&](int h2) {
    return *reinterpret_cast<const u32x4*>(slot + tile_off(t0 + 8 * h2, j));
  };
  auto out_ptr = [&](int64_t i, int h2) {
    return Out + obase + (n_lo + (sub + i * S) * kTile + t0 + 8 * h2) * orow + 8 * j;
  };
  // Main loop over this wave's tiles that lie wholly inside the range: no
  // branches, unconditional stores, the loads of U tiles issued ahead. (The
  // compiler's wait before a tile also covers the stores and loads issued
  // before the loads it needs, so fewer are in flight at that point than U
  // tiles; variants that kept more in flight measured slower.)
  const int64_t whole = two ? (n_hi - n_lo) / kTile : 0;
  const int64_t mine_whole = whole > sub ? (whole - sub + S - 1) / S : 0;
  int64_t i0 = 0;
  {
    for (; i0 + U <= mine_whole; i0 += U) {
#pragma unroll
      for (int u = 0; u < U; ++u) {
        compute(qb[u]);
        // refill qb[u] only after its last use, so it keeps its registers
        __builtin_amdgcn_sched_barrier(0);
        issue(i0 + u + U, qb[u]);
        const u32x4 o0 = out_line(0), o1 = out_line(1);
        wave_lds_order();
        st16_stream(out_ptr(i0 + u, 0), o0);
        st16_stream(out_ptr(i0 + u, 1), o1);
      }
    }
  }
  // Remainder: the last few tiles, the ragged last tile, and a one-head pair.
  for (; i0 < mine; i0 += U) {
#pragma unroll
    for (int u = 0; u < U; ++u) {
      if (i0 + u < mine) {
        compute(qb[u]);
        issue(i0 + u + U, qb[u]);
        const u32x4 o0 = out_line(0), o1 = out_line(1);
        wave_lds_order();
        const int64_t n = n_lo + (sub + (i0 + u) * S) * kTile + t0;
        if (two || j < 4) {
          if (n < n_hi) st16_stream(out_ptr(i0 + u, 0), o0);
          if (n + 8 < n_hi) st16_stream(out_ptr(i0 + u, 1), o1);
        }
      }
    }
  }
}

// ----------------------------------------------------------- fp32 reduce
//
// fp32 blocks hold 2 heads x S sub-streams (wave w: head w%2, sub-stream w/2).

// Sums the S sub-stream accumulators of each head of the block in fixed order
// (sub 0, then 1, 2, ...) into sub-stream 0. All threads of the block must call.
template <int S, int R>
__device__ __forceinline__ void combine_substreams(float (&regs)[R], float* xchg, int hh, int sub) {
  const int l = lane_id();
  if (S > 1) {
    if (sub > 0) {
      float* dst = xchg + ((sub - 1) * 2 + hh) * R * kWave;
#pragma unroll
      for (int r = 0; r < R; ++r) dst[r * kWave + l] = regs[r];
    }
    __syncthreads();
    if (sub == 0) {
      for (int s = 1; s < S; ++s) {
        const float* src = xchg + ((s - 1) * 2 + hh) * R * kWave;
#pragma unroll
        for (int r = 0; r < R; ++r) regs[r] += src[r * kWave + l];
      }
    }
  }
}


// fp32 tiles of the MFMA paths: 32 tokens of one head, 32 channels of 4 bytes
// per token (one 128-byte line). A wave's loads cover whole lines: lane l
// takes 16-byte piece l % 8 of tokens 8 i + l / 8, i < 4.
constexpr int kF32Tile = 32;
constexpr int kF32TileFloats = kF32Tile * kD;  // 1024

// Accumulates phi(K)^T V and phi(K)^T 1 for one head over the tiles sub,
// sub + S, ... of 32 tokens of [n_lo, n_hi), on MFMA 32x32x2 fp32 (exact
// fp32 products, fp32 sums: the fp32 path's accuracy): output row c (K
// channel) and column j (V channel); the k index is the token, two per
// instruction, so both operands are row reads of the staged tiles - lane l
// takes phi(K[2 i + l/32][l%32]) and V[2 i + l/32][l%32]. ksum falls out of
// the same phi(K) values. At the end the sums are handed back in the layout
// of the state helpers: lane l owns state row c = l/2, columns 16*(l%2) ..
// +15 (acc[0..15]), and ksum[c] (acc[16]). slot: the wave's 2 * 1024 floats
// of LDS. Loads are never predicated: a token outside the range reads row
// n_lo and is dropped (phi = 0) when the operands are built.
template <int U, int Fm = kFmapRelu>
__device__ __forceinline__ void reduce_f32_wave(const float* __restrict__ K,
                                                const float* __restrict__ V, int64_t row,
                                                int64_t base, int64_t n_lo, int64_t n_hi,
                                                int sub, int S, float* slot /*2 * 1024*/,
                                                float (&acc)[17]) {
  const int l = lane_id();
  const int lt = l >> 3;        // token lt + 8 i of the tile
  const int lq = l & 7;         // 16-byte piece of the token's line
  const int tk = l >> 5;        // MFMA k: token 2 i + tk
  const int col = l & 31;       // MFMA row (K channel) / column (V channel)
  const int64_t tiles = (n_hi - n_lo + kF32Tile - 1) / kF32Tile;
  const int64_t mine = tiles > sub ? (tiles - sub + S - 1) / S : 0;

  u32x4 kb[U][4], vb[U][4];
  auto issue = [&](int64_t i, u32x4 (&kd)[4], u32x4 (&vd)[4]) {
    const int64_t n0 = n_lo + (sub + i * S) * kF32Tile + lt;
#pragma unroll
    for (int h = 0; h < 4; ++h) {
      const int64_t n = n0 + 8 * h;
      const int64_t off = base + (n < n_hi ? n : n_lo) * row + lq * 4;
      kd[h] = ld16_stream(K + off);
      vd[h] = ld16_stream(V + off);
    }
  };
#pragma unroll
  for (int u = 0; u < U; ++u) issue(u, kb[u], vb[u]);

  float* ks_t = slot;                   // [32 tokens][32 channels]
  float* vs_t = slot + kF32TileFloats;  // [32 tokens][32 channels]
  f32x16 d = (f32x16)0;
  float ksum = 0.0f;
  for (int64_t i0 = 0; i0 < mine; i0 += U) {
#pragma unroll
    for (int u = 0; u < U; ++u) {
      if (i0 + u < mine) {
#pragma unroll
        for (int h = 0; h < 4; ++h) {
          st16(ks_t + (lt + 8 * h) * kD + lq * 4, kb[u][h]);
          st16(vs_t + (lt + 8 * h) * kD + lq * 4, vb[u][h]);
        }
        issue(i0 + u + U, kb[u], vb[u]);
        wave_lds_order();
        const int64_t left = n_hi - (n_lo + (sub + (i0 + u) * S) * kF32Tile);
        const int valid = static_cast<int>(left < kF32Tile ? left : kF32Tile);
        // all operands first, so the LDS reads overlap each other, not the MFMAs
        float av[kF32Tile / 2], bv[kF32Tile / 2];
#pragma unroll
        for (int t2 = 0; t2 < kF32Tile / 2; ++t2) {
          av[t2] = ks_t[(2 * t2 + tk) * kD + col];
          bv[t2] = vs_t[(2 * t2 + tk) * kD + col];
        }
        wave_lds_order();
#pragma unroll
        for (int t2 = 0; t2 < kF32Tile / 2; ++t2) {
          const float a = 2 * t2 + tk < valid ? fmap_f32<Fm>(av[t2]) : 0.0f;
          ksum += a;
          d = __builtin_amdgcn_mfma_f32_32x32x2f32(a, bv[t2], d, 0, 0, 0);
        }
      }
    }
  }
  // back to the state helpers' layout through the slot: [c][33], ksum in column 32
  ksum += __shfl_xor(ksum, 32);
#pragma unroll
  for (int r = 0; r < 16; ++r) slot[(8 * (r >> 2) + 4 * tk + (r & 3)) * kSC + col] = d[r];
  if (l < 32) slot[col * kSC + kD] = ksum;
  wave_lds_order();
  const int c = l >> 1, jh = (l & 1) * 16;
#pragma unroll
  for (int m = 0; m < 16; ++m) acc[m] += slot[c * kSC + jh + m];
  acc[16] += slot[c * kSC + kD];
  wave_lds_order();
}

template <bool Coherent>
__device__ __forceinline__ void store_state_from_f32(float* dst, const float (&acc)[17]) {
  const int l = lane_id();
  const int c = l >> 1;
  const int jh = (l & 1) * 16;
#pragma unroll
  for (int m = 0; m < 16; ++m) put<Coherent>(dst + c * kSC + jh + m, acc[m]);
  if (jh == 0) put<Coherent>(dst + c * kSC + kD, acc[16]);
}

// ------------------------------------------------------------ fp32 apply

constexpr int kPadCols = 36;  // state row padded to 36 floats for 16-byte LDS reads

// Copies a [d][d+1] state (global or LDS) to a padded [d][36] LDS layout.
__device__ __forceinline__ void stage_state_padded(float* dst, const float* st) {
  for (int e = lane_id(); e < kSF; e += kWave) {
    const int c = e / kSC, j = e - c * kSC;
    dst[c * kPadCols + j] = st[e];
  }
}

// LDS of one wave in the fp32 apply: the q tile transposed to [channel][token]
// (row pitch 33 floats, so the operand reads and the staging writes spread
// over the banks), then the output tile [token][channel] (pitch 36 floats,
// 16-byte rows for the line reads), and 1 / den per token.
constexpr int kF32QPitch = 33, kF32OPitch = 36;
constexpr int kF32ApplyU = 2;  // tiles in flight per wave
constexpr int kF32ApplyLds = kF32Tile * kF32OPitch + kF32Tile;  // floats per wave

// Applies one head's state to the tiles sub, sub + S, ... of 32 tokens of
// [n_lo, n_hi) on MFMA 32x32x2 fp32: num (token x output channel) =
// phi(q) KV with k = the q channel, two per instruction - lane l feeds
// phi(q[l%32][2 i + l/32]) and KV[2 i + l/32][l%32], the 16 KV values it
// needs held in registers for the whole range. den = phi(q) . ksum + eps
// from the same phi(q) values (each lane half the channels, the halves
// added by a shuffle). q of token n starts at Q + base + n * row, its output
// at Out + obase + n * orow; stp: the head's state padded to 36 columns in
// LDS; lds: the wave's kF32ApplyLds floats. Tokens past n_hi read row n_lo
// and are not stored.
template <int Fm = kFmapRelu>
__device__ __forceinline__ void apply_f32_wave(const float* __restrict__ Q, float* __restrict__ Out,
                                               const float* stp /*padded LDS*/, float eps,
                                               int64_t row, int64_t base, int64_t orow,
                                               int64_t obase, int64_t n_lo, int64_t n_hi,
                                               int sub, int S, float* lds) {
  const int l = lane_id();
  const int lt = l >> 3, lq = l & 7;
  const int tk = l >> 5, col = l & 31;
  const int64_t tiles = (n_hi - n_lo + kF32Tile - 1) / kF32Tile;
  const int64_t mine = tiles > sub ? (tiles - sub + S - 1) / S : 0;
  float* qt = lds;                        // [32 channels][33]
  float* ot = lds;                        // [32 tokens][36], after qt is consumed
  float* rv = lds + kF32Tile * kF32OPitch;
  float kv[16], ks[16];
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    kv[i] = stp[(2 * i + tk) * kPadCols + col];
    ks[i] = stp[(2 * i + tk) * kPadCols + kD];
  }
  constexpr int U = kF32ApplyU;
  u32x4 qb[U][4];
  auto issue = [&](int64_t i, u32x4 (&qd)[4]) {
    const int64_t n0 = n_lo + (sub + i * S) * kF32Tile + lt;
#pragma unroll
    for (int h = 0; h < 4; ++h) {
      const int64_t n = n0 + 8 * h;
      qd[h] = ld16_stream(Q + base + (n < n_hi ? n : n_lo) * row + lq * 4);
    }
  };
#pragma unroll
  for (int u = 0; u < U; ++u) issue(u, qb[u]);
  for (int64_t i0 = 0; i0 < mine; i0 += U) {
#pragma unroll
    for (int u = 0; u < U; ++u) {
      if (i0 + u < mine) {
        const int64_t tile = sub + (i0 + u) * S;
#pragma unroll
        for (int h = 0; h < 4; ++h) {
          const f32x4 x = __builtin_bit_cast(f32x4, qb[u][h]);
#pragma unroll
          for (int e = 0; e < 4; ++e) qt[(lq * 4 + e) * kF32QPitch + lt + 8 * h] = x[e];
        }
        issue(i0 + u + U, qb[u]);
        wave_lds_order();
        float av[16];
#pragma unroll
        for (int i = 0; i < 16; ++i) av[i] = qt[(2 * i + tk) * kF32QPitch + col];
        wave_lds_order();
        f32x16 d = (f32x16)0;
        float den = 0.0f;
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const float a = fmap_f32<Fm>(av[i]);
          den = __builtin_fmaf(a, ks[i], den);
          d = __builtin_amdgcn_mfma_f32_32x32x2f32(a, kv[i], d, 0, 0, 0);
        }
        den += __shfl_xor(den, 32);
        if (l < 32) rv[col] = 1.0f / (den + eps);
        wave_lds_order();
        // d lane l, register r: token 8 (r / 4) + 4 (l / 32) + r % 4, channel l % 32
        f32x4 r4[4];
#pragma unroll
        for (int g = 0; g < 4; ++g)
          r4[g] = *reinterpret_cast<const f32x4*>(rv + 8 * g + 4 * tk);
#pragma unroll
        for (int r = 0; r < 16; ++r)
          ot[(8 * (r >> 2) + 4 * tk + (r & 3)) * kF32OPitch + col] = d[r] * r4[r >> 2][r & 3];
        wave_lds_order();
        const int64_t n0 = n_lo + tile * kF32Tile + lt;
#pragma unroll
        for (int h = 0; h < 4; ++h) {
          const u32x4 o = *reinterpret_cast<const u32x4*>(ot + (lt + 8 * h) * kF32OPitch + lq * 4);
          if (n0 + 8 * h < n_hi) st16(Out + obase + (n0 + 8 * h) * orow + lq * 4, o);
        }
        wave_lds_order();
      }
    }
  }
}

// ---------------------------------------------------------------- kernels

struct BlockCoords {
  int64_t b, h, p;
  int hh, sub;
  bool active;
};

__device__ __forceinline__ BlockCoords block_coords(int64_t pairs, int64_t units, int64_t H) {
  BlockCoords c;
  const int64_t bid = blockIdx.x;
  const int64_t unit = bid % units;
  c.p = bid / units;
  c.b = unit / pairs;
  // the wave index is uniform across the wave; say so, so that loop control
  // derived from it stays scalar
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  c.hh = w & 1;
  c.sub = w >> 1;
  c.h = 2 * (unit % pairs) + c.hh;
  c.active = c.h < H;
  return c;
}

// bf16 blocks: S waves, all on one head pair; wave w is token sub-stream w.
struct PairCoords {
  int64_t b, h, p;
  int sub;
  bool two;  // the pair's second head exists
};

// Block g of a one-block-per-unit grid.
__device__ __forceinline__ PairCoords pair_coords(int64_t pairs, int64_t H) {
  PairCoords c;
  const int64_t unit = blockIdx.x;
  c.p = 0;
  c.b = unit / pairs;
  c.h = 2 * (unit % pairs);
  c.sub = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  c.two = c.h + 1 < H;
  return c;
}

// LDS of a bf16 reduction block: one K + V tile slot per wave, reused at the
// end of each head pair's range to fold the waves' sums (34 floats per lane).
constexpr int kFoldFloats = 34;  // 32 accumulator registers + ksum of both heads
template <int S>
union alignas(16) RedLds {
  unsigned char slot[S][2 * kTileBytes];
  float xchg[S][kFoldFloats][kWave];
};

// Block epilogue of the bf16 reduction: every wave writes its sums for the
// head pair (acc in the 32x32 MFMA layout, ks per lane) to LDS; after one
// barrier the whole block adds them in wave order and writes the pair's
// [2][d][d+1] state to dst (only the first head when !two).
// 32x32 accumulator layout: lane l, register r holds row
// 8*(r/4) + 4*(l/32) + r%4 and column l%32; rows are k channels c, columns
// v channels j. ksum[c] is ks of lane c plus ks of lane c + 32 (the two
// token halves of the gather), added in that order.
// The KV part (2 x 32 x 32 values) is spread evenly over the block, each
// thread issuing all its LDS reads before its first add; the 64 ksum values
// go to the first 64 threads as one more batch. (A loop over the [d][d+1]
// rows instead puts a ksum element in almost every wave, whose divergent
// second path doubled the epilogue.)
template <int S, bool Coherent>
__device__ __forceinline__ void block_sum_state(const f32x16 (&acc)[2], const float (&ks)[2],
                                                float (&xchg)[S][kFoldFloats][kWave], int sub,
                                                float* dst, bool two) {
  static_assert(2 * kD * kD % (kWave * S) == 0, "KV values split evenly over the block");
  constexpr int kPer = 2 * kD * kD / (kWave * S);  // KV values per thread
  const int l = lane_id();
  __syncthreads();  // every wave is done with its tile slot (xchg overlays them)
#pragma unroll
  for (int r = 0; r < 16; ++r) {
    xchg[sub][r][l] = acc[0][r];
    xchg[sub][16 + r][l] = acc[1][r];
  }
  xchg[sub][32][l] = ks[0];
  xchg[sub][33][l] = ks[1];
  __syncthreads();
  const int heads = two ? 2 : 1;
  float x[kPer][S];
#pragma unroll
  for (int i = 0; i < kPer; ++i) {
    const int m = threadIdx.x + i * kWave * S;  // (head, c, j) = (m >> 10, (m >> 5) & 31, m & 31)
    const int c = (m >> 5) & 31, j = m & 31;
    const int r = 16 * (m >> 10) + 4 * (c >> 3) + (c & 3);
    const int ln = j + 32 * ((c >> 2) & 1);
#pragma unroll
    for (int w = 0; w < S; ++w) x[i][w] = xchg[w][r][ln];
  }
#pragma unroll
  for (int i = 0; i < kPer; ++i) {
    const int m = threadIdx.x + i * kWave * S;
    float sum = x[i][0];
#pragma unroll
    for (int w = 1; w < S; ++w) sum += x[i][w];
    if ((m >> 10) < heads) put<Coherent>(dst + (m >> 10) * kSF + ((m >> 5) & 31) * kSC + (m & 31), sum);
  }
  if (threadIdx.x < 2 * kD) {
    const int hh = threadIdx.x >> 5, c = threadIdx.x & 31;
    float y[S][2];
#pragma unroll
    for (int w = 0; w < S; ++w) {
      y[w][0] = xchg[w][32 + hh][c];
      y[w][1] = xchg[w][32 + hh][c + 32];
    }
    float sum = y[0][0] + y[0][1];
#pragma unroll
    for (int w = 1; w < S; ++w) sum += y[w][0] + y[w][1];
    if (hh < heads) put<Coherent>(dst + hh * kSF + c * kSC + kD, sum);
  }
}

// Balanced ranges. The work of a bf16 kernel is the flattened index
// f = unit * T + t over head-pair units (b, pair) and their T 16-token tiles.
// Block g takes f in [g * Qb, (g + 1) * Qb): one round of co-resident blocks,
// equal shares, crossing unit boundaries where they fall. Within a unit's
// segment the block's S waves take its tiles as interleaved sub-streams.
struct Segment {
  int64_t unit, b, h, n_lo, n_hi;
  bool two;
};

__device__ __forceinline__ Segment segment_of(int64_t unit, int64_t f_lo, int64_t f_hi, int64_t T,
                                              int64_t N, int64_t H, int64_t pairs) {
  Segment sg;
  sg.unit = unit;
  sg.b = unit / pairs;
  sg.h = 2 * (unit % pairs);
  sg.two = sg.h + 1 < H;
  const int64_t t_lo = (f_lo > unit * T ? f_lo : unit * T) - unit * T;
  const int64_t t_hi = (f_hi < (unit + 1) * T ? f_hi : (unit + 1) * T) - unit * T;
  sg.n_lo = t_lo * kTile;
  sg.n_hi = t_hi * kTile < N ? t_hi * kTile : N;
  return sg;
}

// The blocks of the reduction that touch unit `unit` when block g covers
// tiles [g * Qb, (g + 1) * Qb) of the flattened (unit, tile) index: blocks
// first .. first + count - 1. Block g writes the unit's partial g - first.
struct SlotRange {
  int64_t first, count;
};
__device__ __forceinline__ SlotRange slot_range(int64_t unit, int64_t T, int64_t Qb) {
  const int64_t first = unit * T / Qb;
  return {first, ((unit + 1) * T - 1) / Qb - first + 1};
}

// Partial slots a unit's state is split into, by the rule `Qr` of the grid
// that wrote them: Qr > 0, balanced ranges of Qr tiles (slot_range); Qr < 0,
// a (unit, chunk) grid of -Qr chunks per unit, one slot per chunk; Qr = 0, a
// single folded state.
__device__ __forceinline__ int64_t slot_count(int64_t unit, int64_t T, int64_t Qr) {
  return Qr > 0 ? slot_range(unit, T, Qr).count : (Qr < 0 ? -Qr : 1);
}

// XCD-grouped (unit, chunk) items. The hardware deals blocks to the XCDs
// round robin (block g to XCD g % X on MI355X, X = 8), and each XCD has its
// own L2. The units * C items, unit-major, are cut into X contiguous runs of
// `per` = ceil(units * C / X) items; block g takes item g / X of run g % X.
// Every XCD then gets the same number of blocks, and a unit's chunk blocks
// share one L2 (or two, where a run boundary splits the unit), which fetches
// the unit's partials about once instead of once per block. The grid is
// X * per blocks; the few past the last item exit. X = 1 keeps the plain
// order; the mapping is a bijection either way, only locality depends on X.
struct Item {
  int64_t unit, chunk;
  bool valid;
};
__device__ __forceinline__ Item xcd_item(int64_t units, int64_t C, int64_t X) {
  const int64_t items = units * C;
  const int64_t per = (items + X - 1) / X;
  const int64_t item = (blockIdx.x % X) * per + blockIdx.x / X;
  const int64_t unit = item / C;
  return {unit, item - unit * C, item < items};
}

// State reduction over one block's range. For each unit it touches, the
// block folds its waves' sums and writes them as partial number
// (g - first block of the unit) of that unit. With Fold, the last of the
// unit's contributing blocks also folds the unit's partials, in order, into
// the state; without, the partials are the result (the apply sums them).
// Partials: [units][slots][2 heads][d][d+1]. Element (b, n, h, c) of k and
// v is at b * N * ld + n * ld + h * d + c (ld = H * d when contiguous).
// KeepK: k is read with ordinary loads instead of streaming ones, for a
// caller that reads it again after a pass over other tensors (the
// backward's k/v pass).
template <int S, int U, bool Fold, int Fm = kFmapRelu, bool KeepK = false>
__global__ __launch_bounds__(64 * S) void reduce_bf16_kernel(
    const unsigned short* __restrict__ K, const unsigned short* __restrict__ V,
    float* __restrict__ partials, float* __restrict__ state, unsigned long long* __restrict__ ctl,
    unsigned long long epoch, int64_t N, int64_t H, int64_t ld, int64_t pairs, int64_t T,
    int64_t Qb, int64_t F, int64_t slots, int64_t C, int64_t X) {
  __shared__ RedLds<S> lds;
  const int sub = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int64_t g = blockIdx.x;
  // C > 0: (unit, chunk) items of Qb tiles, C = ceil(T / Qb) chunks per unit,
  // in XCD runs (xcd_item); the chunk is the slot. C = 0: balanced ranges.
  int64_t f_lo, f_hi, chunk = 0;
  if (C > 0) {
    const Item it = xcd_item(F / T, C, X);
    if (!it.valid) return;  // the whole block
    chunk = it.chunk;
    f_lo = it.unit * T + it.chunk * Qb;
    f_hi = f_lo + Qb < (it.unit + 1) * T ? f_lo + Qb : (it.unit + 1) * T;
  } else {
    f_lo = g * Qb;
    f_hi = f_lo + Qb < F ? f_lo + Qb : F;
  }
  for (int64_t unit = f_lo / T; unit * T < f_hi; ++unit) {
    const Segment sg = segment_of(unit, f_lo, f_hi, T, N, H, pairs);
    const int64_t base = sg.b * N * ld + sg.h * kD;
    f32x16 acc[2] = {(f32x16)0, (f32x16)0};
    float ks[2] = {0.0f, 0.0f};
    reduce_pair_wave<U, Fm, KeepK>(K, V, ld, base, sg.n_lo, sg.n_hi, sub, S, sg.two,
                                   lds.slot[sub], acc, ks);
    int64_t slot, count;
    if (C > 0) {
      slot = chunk;
      count = C;
    } else {
      const SlotRange sr = slot_range(unit, T, Qb);
      slot = g - sr.first;
      count = sr.count;
    }
    float* part = partials + ((unit * slots) + slot) * 2 * kSF;
    block_sum_state<S, Fold>(acc, ks, lds.xchg, sub, part, sg.two);
    if (Fold && arrive_last(ctl + unit, epoch, count))
      fold_partials(partials + unit * slots * 2 * kSF, 2 * kSF, state + (sg.b * H + sg.h) * kSF,
                    (sg.two ? 2 : 1) * kSF, count);
    __syncthreads();  // the LDS is reused by the next segment
  }
}

template <int S, int U, int Fm = kFmapRelu>
__global__ __launch_bounds__(128 * S) void reduce_f32_kernel(
    const float* __restrict__ K, const float* __restrict__ V, float* __restrict__ partials,
    float* __restrict__ state, unsigned long long* __restrict__ ctl, unsigned long long epoch,
    int64_t N, int64_t H, int64_t ld, int64_t pairs, int64_t units, int64_t chunk,
    int64_t nchunks, int64_t BH) {
  __shared__ alignas(16) float slot[2 * S][2 * kF32TileFloats];
  __shared__ float xchg[(S > 1 ? S - 1 : 1) * 2 * 17 * kWave];
  const BlockCoords bc = block_coords(pairs, units, H);
  const int64_t n_lo = bc.p * chunk;
  const int64_t n_hi = n_lo + chunk < N ? n_lo + chunk : N;
  float acc[17];
#pragma unroll
  for (int r = 0; r < 17; ++r) acc[r] = 0.0f;
  if (bc.active)
    reduce_f32_wave<U, Fm>(K, V, ld, bc.b * N * ld + bc.h * kD, n_lo, n_hi, bc.sub, S,
                           slot[threadIdx.x >> 6], acc);
  combine_substreams<S, 17>(acc, xchg, bc.hh, bc.sub);
  if (bc.active && bc.sub == 0)
    store_state_from_f32<true>(partials + (bc.p * BH + bc.b * H + bc.h) * kSF, acc);
  const int64_t unit = blockIdx.x % units;
  if (arrive_last(ctl + unit, epoch, nchunks)) {
    const int64_t bh0 = bc.b * H + 2 * (unit % pairs);
    fold_partials(partials + bh0 * kSF, BH * kSF, state + bh0 * kSF,
                  (H - 2 * (unit % pairs) < 2 ? 1 : 2) * kSF, nchunks);
  }
}

// The state of one head pair as the sum of `count` consecutive
// [2][d][d+1] fp32 slots at st (slot stride 2 * kSF floats), written to
// stage (n4 = (heads) * kSF / 4 float4s). Slot 0 starts each sum, later slots
// add in ascending order - the order fold_partials uses. Each thread sums
// elements e and e + blockDim.x (blockDim.x >= n4 / 2); loads are
// unconditional (indices clamped to valid slots and elements) and a batch's
// loads are all issued before any is added. The caller synchronises before
// reading stage.
// The first kFirstSlots slots of such a sum, loaded ahead (indices clamped
// to valid slots and elements), so a caller can issue them before its other
// loads: a wave's loads complete in issue order, so the sum then waits for
// these alone.
constexpr int kFirstSlots = 4;
struct SlotPrefetch {
  f32x4 x0[kFirstSlots], x1[kFirstSlots];
};
__device__ __forceinline__ SlotPrefetch prefetch_slots(const f32x4* __restrict__ st,
                                                       int64_t count, int n4) {
  const int e0 = threadIdx.x < n4 ? threadIdx.x : n4 - 1;
  const int e1 = threadIdx.x + blockDim.x < n4 ? threadIdx.x + blockDim.x : n4 - 1;
  SlotPrefetch pf;
#pragma unroll
  for (int u = 0; u < kFirstSlots; ++u) {
    const int64_t j = u < count ? u : count - 1;
    pf.x0[u] = st[j * (2 * kSF / 4) + e0];
    pf.x1[u] = st[j * (2 * kSF / 4) + e1];
  }
  return pf;
}

__device__ __forceinline__ void sum_slots_to_lds(const f32x4* __restrict__ st, int64_t count,
                                                 int n4, f32x4* stage, const SlotPrefetch& pf) {
  constexpr int kBatch = 8;
  const int e0 = threadIdx.x < n4 ? threadIdx.x : n4 - 1;
  const int e1 = threadIdx.x + blockDim.x < n4 ? threadIdx.x + blockDim.x : n4 - 1;
  f32x4 a0 = pf.x0[0], a1 = pf.x1[0];
#pragma unroll
  for (int u = 1; u < kFirstSlots; ++u) {
    a0 = u < count ? a0 + pf.x0[u] : a0;
    a1 = u < count ? a1 + pf.x1[u] : a1;
  }
  for (int64_t j0 = kFirstSlots; j0 < count; j0 += kBatch) {
    f32x4 x0[kBatch], x1[kBatch];
#pragma unroll
    for (int u = 0; u < kBatch; ++u) {
      const int64_t j = min(j0 + u, count - 1);
      x0[u] = st[j * (2 * kSF / 4) + e0];
      x1[u] = st[j * (2 * kSF / 4) + e1];
    }
#pragma unroll
    for (int u = 0; u < kBatch; ++u) {
      const bool take = j0 + u < count;
      a0 = take ? a0 + x0[u] : a0;
      a1 = take ? a1 + x1[u] : a1;
    }
  }
  if (threadIdx.x < n4) stage[threadIdx.x] = a0;
  if (threadIdx.x + blockDim.x < n4) stage[threadIdx.x + blockDim.x] = a1;
}
__device__ __forceinline__ void sum_slots_to_lds(const f32x4* __restrict__ st, int64_t count,
                                                 int n4, f32x4* stage) {
  sum_slots_to_lds(st, count, n4, stage, prefetch_slots(st, count, n4));
}


// Apply, one block per (unit, token chunk of Qa tiles), C chunks per unit,
// grouped by XCD (xcd_item), or balanced ranges (C = 0).
// The state of a unit is the sum of `count`
// consecutive [2][d][d+1] slots at src + b * sb + p * sp (+ j * 2 * kSF),
// count = slot_count(unit, T, Qr): the partials of the reduction (balanced
// ranges or a (unit, chunk) grid), summed here in ascending slot order, as
// fold_partials does; a fixed number of slots per unit; or 1, a folded state.
// The block sums them once into LDS; each wave then builds
// its MFMA operands from there. q has token stride ld (as k and v in
// reduce_bf16_kernel); the output is contiguous [B][N][H][d].
template <int S, int U, int Fm = kFmapRelu>
__global__ __launch_bounds__(64 * S) void apply_bf16_kernel(
    const unsigned short* __restrict__ Q, const float* __restrict__ src, int64_t sb, int64_t sp,
    int64_t Qr, unsigned short* __restrict__ Out, float eps, int64_t N, int64_t H, int64_t ld,
    int64_t pairs, int64_t units, int64_t T, int64_t C, int64_t Qa, int64_t X) {
  static_assert(2 * kWave * S >= 2 * kSF / 4, "two state elements per thread cover a pair");
  __shared__ alignas(16) unsigned char slots[S][kTileBytes];
  __shared__ f32x4 stage[2 * kSF / 4];
  const int sub = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  // C > 0: one (unit, chunk) item of Qa tiles per block, in XCD runs.
  // C = 0: balanced ranges of Qa tiles of the flattened (unit, tile) index;
  // a block that straddles units applies each in turn.
  int64_t f_lo, f_hi;
  if (C > 0) {
    const Item it = xcd_item(units, C, X);
    if (!it.valid) return;  // the whole block
    f_lo = it.unit * T + it.chunk * Qa;
    f_hi = f_lo + Qa < (it.unit + 1) * T ? f_lo + Qa : (it.unit + 1) * T;
  } else {
    f_lo = static_cast<int64_t>(blockIdx.x) * Qa;
    f_hi = f_lo + Qa < units * T ? f_lo + Qa : units * T;
  }
  for (int64_t unit = f_lo / T; unit * T < f_hi; ++unit) {
    const Segment sg = segment_of(unit, f_lo, f_hi, T, N, H, pairs);
    const int64_t count = slot_count(unit, T, Qr);
    const f32x4* st = reinterpret_cast<const f32x4*>(src + sg.b * sb + (sg.h >> 1) * sp);
    const int n4 = (sg.two ? 2 : 1) * kSF / 4;
    auto pre_ops = [&] { return prefetch_slots(st, count, n4); };
    auto make_ops = [&](ApplyOperands (&op)[2], const SlotPrefetch& pf) {
      sum_slots_to_lds(st, count, n4, stage, pf);
      __syncthreads();
      const float* stf = reinterpret_cast<const float*>(stage);
      op[0] = make_apply_operands(stf);
      op[1] = sg.two ? make_apply_operands(stf + kSF) : op[0];
    };
    apply_pair_wave<U, Fm>(Q, Out, pre_ops, make_ops, eps, ld, sg.b * N * ld + sg.h * kD, H * kD,
                           (sg.b * N * H + sg.h) * kD, sg.n_lo, sg.n_hi, sub, S, sg.two,
                           slots[sub]);
    __syncthreads();  // every wave has its operands before `stage` is refilled
  }
}

template <int S, int Fm = kFmapRelu>
__global__ __launch_bounds__(128 * S) void apply_f32_kernel(
    const float* __restrict__ Q, const float* __restrict__ state, float* __restrict__ Out,
    float eps, int64_t N, int64_t H, int64_t ld, int64_t pairs, int64_t units, int64_t chunk) {
  __shared__ float stp[2][kD * kPadCols];
  __shared__ alignas(16) float wl[2 * S][kF32ApplyLds];
  const BlockCoords bc = block_coords(pairs, units, H);
  if (bc.active && bc.sub == 0) stage_state_padded(stp[bc.hh], state + (bc.b * H + bc.h) * kSF);
  __syncthreads();
  if (!bc.active) return;
  const int64_t n_lo = bc.p * chunk;
  const int64_t n_hi = n_lo + chunk < N ? n_lo + chunk : N;
  apply_f32_wave<Fm>(Q, Out, stp[bc.hh], eps, ld, bc.b * N * ld + bc.h * kD, H * kD,
                     (bc.b * N * H + bc.h) * kD, n_lo, n_hi, bc.sub, S, wl[threadIdx.x >> 6]);
}

// One block per (b, head pair) over all N tokens: reduce into registers,
// fold the sub-streams through LDS, keep the state in LDS, apply.
template <int S, int U>
__global__ __launch_bounds__(64 * S) void fused_bf16_kernel(
    const unsigned short* __restrict__ Q, const unsigned short* __restrict__ K,
    const unsigned short* __restrict__ V, unsigned short* __restrict__ Out, float eps,
    int64_t N, int64_t H, int64_t pairs) {
  __shared__ RedLds<S> lds;
  __shared__ float st[2][kSF];
  const PairCoords pc = pair_coords(pairs, H);
  const int64_t base = (pc.b * N * H + pc.h) * kD;
  f32x16 acc[2] = {(f32x16)0, (f32x16)0};
  float ks[2] = {0.0f, 0.0f};
  reduce_pair_wave<U>(K, V, H * kD, base, 0, N, pc.sub, S, pc.two, lds.slot[pc.sub], acc, ks);
  auto pre_ops = [] { return 0; };
  auto make_ops = [&](ApplyOperands (&op)[2], int) {
    // both heads, also for a one-head pair (its second head is never stored)
    block_sum_state<S, false>(acc, ks, lds.xchg, pc.sub, &st[0][0], true);
    __syncthreads();  // the state is complete; xchg is free for the tile slots
    op[0] = make_apply_operands(st[0]);
    op[1] = make_apply_operands(st[1]);
  };
  apply_pair_wave<U>(Q, Out, pre_ops, make_ops, eps, H * kD, base, H * kD, base, 0, N, pc.sub, S,
                     pc.two, lds.slot[pc.sub]);
}

template <int S, int U>
__global__ __launch_bounds__(128 * S) void fused_f32_kernel(
    const float* __restrict__ Q, const float* __restrict__ K, const float* __restrict__ V,
    float* __restrict__ Out, float eps, int64_t N, int64_t H, int64_t pairs) {
  __shared__ alignas(16) float slot[2 * S][2 * kF32TileFloats];
  __shared__ float xchg[(S > 1 ? S - 1 : 1) * 2 * 17 * kWave];
  __shared__ float st[2][kSF];
  __shared__ float stp[2][kD * kPadCols];
  const BlockCoords bc = block_coords(pairs, (int64_t)gridDim.x, H);
  const int64_t base = (bc.b * N * H + bc.h) * kD;
  float acc[17];
#pragma unroll
  for (int r = 0; r < 17; ++r) acc[r] = 0.0f;
  if (bc.active)
    reduce_f32_wave<U>(K, V, H * kD, base, 0, N, bc.sub, S, slot[threadIdx.x >> 6], acc);
  combine_substreams<S, 17>(acc, xchg, bc.hh, bc.sub);
  if (bc.active && bc.sub == 0) store_state_from_f32<false>(st[bc.hh], acc);
  __syncthreads();
  if (bc.active && bc.sub == 0) stage_state_padded(stp[bc.hh], st[bc.hh]);
  __syncthreads();
  if (!bc.active) return;
  apply_f32_wave(Q, Out, stp[bc.hh], eps, H * kD, base, H * kD, base, 0, N, bc.sub, S,
                 slot[threadIdx.x >> 6]);
}

// ------------------------------------------------------------ bf16 backward
//
// Gradients of the forward pass, per head (S_aug = [S | z], g = dL/dout):
//   dnum_i = g_i / den_i,  dden_i = -(g_i . num_i) / den_i^2
//   dq_i   = ([S | z] [dnum_i | dden_i]^T) * [q_i > 0]
//   [dS | dz] = sum_i phi(q_i)^T [dnum_i | dden_i]
//   dk_n   = ([dS | dz] [v_n | 1]^T) * [k_n > 0],   dv_n = phi(k_n) dS
// bwd_q reads q and g, writes dq and per-block [dS | dz] partials (its token
// reduction has the forward reduction's grid and epilogue); bwd_kv reads k,
// v and those partials and writes dk and dv (the apply's grid). Both build
// their state from the sum of partials, like the apply.

// A operands of 16x16x32 MFMAs computing y = M x for a [d][d+1] fp32 matrix
// M (first d columns) and one length-d vector x per token, x in the B
// operand (k = 8*(l/16) + s, token l%16). Row i of tile t stands for
// channel 8*(i/4) + 4t + i%4 (make_apply_operands's permutation), so after
// the two tiles a lane holds y for channels 8*(l/16) .. +7 of token l%16.
// M's last column for those 8 channels rides along for the VALU.
struct RowOperands {
  bf16x8 m0_hi, m0_lo, m1_hi, m1_lo;
  float last[8];
};

__device__ __forceinline__ RowOperands make_row_operands(const float* st) {
  const int l = lane_id();
  const int g = l >> 4;
  const int i = l & 15;
  RowOperands o;
#pragma unroll
  for (int s = 0; s < 8; ++s) {
    const int k = 8 * g + s;
    const float x0 = st[(8 * (i >> 2) + (i & 3)) * kSC + k];
    const float x1 = st[(8 * (i >> 2) + 4 + (i & 3)) * kSC + k];
    const __bf16 h0 = (__bf16)x0, h1 = (__bf16)x1;
    o.m0_hi[s] = h0;
    o.m0_lo[s] = (__bf16)(x0 - (float)h0);
    o.m1_hi[s] = h1;
    o.m1_lo[s] = (__bf16)(x1 - (float)h1);
  }
#pragma unroll
  for (int m = 0; m < 8; ++m) o.last[m] = st[(8 * g + m) * kSC + kD];
  return o;
}

// y = M x for the lane's 8 channels. x is exact in bf16 (x_hi, no x_lo) or
// fp32 split as x_hi + x_lo; the products keep M's hi and lo parts.
template <bool SplitX>
__device__ __forceinline__ void row_product(const RowOperands& o, bf16x8 x_hi, bf16x8 x_lo,
                                            float (&y)[8]) {
  f32x4 e0 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(o.m0_hi, x_hi, (f32x4)0, 0, 0, 0);
  e0 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(o.m0_lo, x_hi, e0, 0, 0, 0);
  f32x4 e1 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(o.m1_hi, x_hi, (f32x4)0, 0, 0, 0);
  e1 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(o.m1_lo, x_hi, e1, 0, 0, 0);
  if (SplitX) {
    e0 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(o.m0_hi, x_lo, e0, 0, 0, 0);
    e1 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(o.m1_hi, x_lo, e1, 0, 0, 0);
  }
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    y[r] = e0[r];
    y[4 + r] = e1[r];
  }
}

// y = phi(x) M for the lane's 8 output channels (the forward apply's
// numerator, no normaliser): 4 MFMAs with M^T's hi and lo parts.
__device__ __forceinline__ void col_product(const ApplyOperands& op, bf16x8 px, float (&y)[8]) {
  f32x4 a0 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(op.kv0_hi, px, (f32x4)0, 0, 0, 0);
  a0 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(op.kv0_lo, px, a0, 0, 0, 0);
  f32x4 a1 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(op.kv1_hi, px, (f32x4)0, 0, 0, 0);
  a1 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(op.kv1_lo, px, a1, 0, 0, 0);
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    y[r] = a0[r];
    y[4 + r] = a1[r];
  }
}

// Sum over the 4 lanes that hold one token's 32 channels (l, l^16, l^32, l^48).
// (gfx950's permlane16/32_swap would avoid the LDS round trip, but this
// compiler folds the builtin's two results of a swap of x with itself into
// one register, and the same swaps written as inline assembly gave sums that
// differ from the shuffles' on the GPU; the shuffles are kept.)
__device__ __forceinline__ float token_sum(float x) {
  x += __shfl_xor(x, 16);
  x += __shfl_xor(x, 32);
  return x;
}

// LDS of one wave in bwd_q: the q and g tiles (whole lines, swizzled as in
// the forward) and, for one head, the 1 / den and dden rows of the tile.
// 16-byte alignment is stated so the 16-byte accesses stay single
// ds_read/write_b128 instructions: at 4-byte alignment the compiler splits
// them into 8-byte pairs, whose 16-byte lane stride conflicts 4 ways.
struct alignas(16) BwdQWaveLds {
  unsigned char q[kTileBytes];
  unsigned char g[kTileBytes];
  float rv[kTile];
  float dd[kTile];
};

// bwd_q for the pair's two heads over the tiles sub, sub + S, ... of
// [n_lo, n_hi): writes dq, and adds phi(q)^T dnum (acc, 32x32 MFMA layout)
// and phi(q)^T dden (ks, per lane: channel l%32 over the lane's 8 tokens)
// for the pair. make_ops(ro) fills the state's operands once the first
// loads are out. One product per token carries the step: with u = S g,
// g . num = phi(q) . u (num = phi(q) S), and since dnum = g / den,
// S dnum = u / den, so dphi(q) = u / den + z dden. den = phi(q) . z + eps is
// summed on the VALU from z. The token reduction uses the same fact:
// phi(q)^T dnum = (phi(q) / den)^T g, so the 32x32x16 MFMA takes g exactly
// (gathered from the g tile) and phi(q) / den split into bf16 hi + lo.
// Padded tokens (n >= n_hi) read row n_lo, are zeroed in the q tile and get
// 1 / den = dden = 0, so they add nothing even where eps = 0.
template <int U, int Fm, class MakeOps>
__device__ __forceinline__ void grad_q_pair_wave(const unsigned short* __restrict__ Q,
                                                 const unsigned short* __restrict__ G,
                                                 unsigned short* __restrict__ dQ,
                                                 MakeOps&& make_ops, float eps, int64_t row,
                                                 int64_t base, int64_t n_lo, int64_t n_hi,
                                                 int sub, int S, bool two, BwdQWaveLds& w,
                                                 f32x16 (&acc)[2], float (&ks)[2]) {
  const int l = lane_id();
  const int t0 = l >> 3;
  const int j = l & 7;
  const int jl = two ? j : (j & 3);
  const int g = l >> 4;
  const int col = l & 15;
  const int rt = (l >> 5) * 8;
  const int64_t tiles = (n_hi - n_lo + kTile - 1) / kTile;
  const int64_t mine = tiles > sub ? (tiles - sub + S - 1) / S : 0;

  u32x4 qb[U][2], gb[U][2];
  auto issue = [&](int64_t i, u32x4 (&qd)[2], u32x4 (&gd)[2]) {
    const int64_t n0 = n_lo + (sub + i * S) * kTile + t0;
#pragma unroll
    for (int h2 = 0; h2 < 2; ++h2) {
      const int64_t n = n0 + 8 * h2;
      const int64_t off = base + (n < n_hi ? n : n_lo) * row + 8 * jl;
      qd[h2] = ld16_stream(Q + off);
      gd[h2] = ld16_stream(G + off);
    }
  };
#pragma unroll
  for (int u = 0; u < U; ++u) issue(u, qb[u], gb[u]);
  RowOperands ro[2];
  make_ops(ro);

  // stage() moves a tile's lines from registers to LDS; the registers then
  // take the next tile's loads, which stay in flight while compute() works
  // from LDS. (Issuing them after compute instead, as the memory-bound
  // passes do, measured 2.4 us slower here.)
  auto stage = [&](int64_t i, const u32x4 (&qin)[2], const u32x4 (&gin)[2]) {
    const int64_t n0 = n_lo + (sub + i * S) * kTile;
#pragma unroll
    for (int h2 = 0; h2 < 2; ++h2) {
      const int o = tile_off(t0 + 8 * h2, j);
      *reinterpret_cast<u32x4*>(w.q + o) = n0 + t0 + 8 * h2 < n_hi ? qin[h2] : (u32x4)0;
      *reinterpret_cast<u32x4*>(w.g + o) = gin[h2];
    }
    wave_lds_order();
  };
  auto compute = [&](int64_t i) {
    const int64_t n0 = n_lo + (sub + i * S) * kTile;
    const bool valid = n0 + col < n_hi;
#pragma unroll
    for (int hh = 0; hh < 2; ++hh) {
      const int po = tile_off(col, hh * 4 + g);
      const u32x4 qraw = *reinterpret_cast<const u32x4*>(w.q + po);
      const u32x4 graw = *reinterpret_cast<const u32x4*>(w.g + po);
      float pq[8], u[8], dph[8];
      const u32x4 rq = relu_bf16x8(qraw);
      if (Fm == kFmapRelu) {
        widen_bf16x8(rq, pq);
      } else {
        // phi(q) and phi'(q) in fp32 (a padded token's zeroed q gives
        // finite values, and its 1 / den and dden of 0 keep it out)
        widen_bf16x8(qraw, pq);
#pragma unroll
        for (int m = 0; m < 8; ++m) fmap_dfmap_hw<Fm>(pq[m], pq[m], dph[m]);
      }
      row_product<false>(ro[hh], __builtin_bit_cast(bf16x8, graw), (bf16x8)0, u);  // u = S g
      float dp = 0.0f, p = 0.0f;
#pragma unroll
      for (int m = 0; m < 8; ++m) {
        dp += pq[m] * ro[hh].last[m];  // phi(q) . z over the lane's channels
        p += pq[m] * u[m];             // g . num = phi(q) . (S g)
      }
      const float rinv = __builtin_amdgcn_rcpf(token_sum(dp) + eps);  // 1 ulp
      p = token_sum(p);
      const float dden = valid ? -p * rinv * rinv : 0.0f;
      // dq for the lane's channels: S dnum + z dden = u / den + z dden, then the ReLU gate
      u32x4 dqw;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const float d0 = u[2 * e] * rinv + ro[hh].last[2 * e] * dden;
        const float d1 = u[2 * e + 1] * rinv + ro[hh].last[2 * e + 1] * dden;
        dqw[e] = Fm == kFmapRelu ? relu_gate_pk(cvt_pk_bf16(d0, d1), rq[e])
                                 : cvt_pk_bf16(d0 * dph[2 * e], d1 * dph[2 * e + 1]);
      }
      const bf16x8 dq = __builtin_bit_cast(bf16x8, dqw);
      // the token reduction: 1 / den and dden rows to LDS, the operands
      // gathered transposed (k = the lane's 8 tokens, channel l%32)
      if (g == 0) {
        w.rv[col] = valid ? rinv : 0.0f;
        w.dd[col] = dden;
      }
      wave_lds_order();
      const s16x8 a = gather_tokens8(w.q, hh);
      const s16x8 b = gather_tokens8(w.g, hh);
      const f32x4 rv0 = *reinterpret_cast<const f32x4*>(w.rv + rt);
      const f32x4 rv1 = *reinterpret_cast<const f32x4*>(w.rv + rt + 4);
      const f32x4 dd0 = *reinterpret_cast<const f32x4*>(w.dd + rt);
      const f32x4 dd1 = *reinterpret_cast<const f32x4*>(w.dd + rt + 4);
      wave_lds_order();
      float pf[8], sc[8];
      if (Fm == kFmapRelu) {
        widen_bf16x8(relu_bf16x8(__builtin_bit_cast(u32x4, a)), pf);
      } else {
        widen_bf16x8(__builtin_bit_cast(u32x4, a), pf);
#pragma unroll
        for (int s = 0; s < 8; ++s) pf[s] = fmap_hw<Fm>(pf[s]);
      }
      float zs = 0.0f;
#pragma unroll
      for (int s = 0; s < 4; ++s) {
        sc[s] = pf[s] * rv0[s];
        sc[4 + s] = pf[4 + s] * rv1[s];
        zs += pf[s] * dd0[s];
        zs += pf[4 + s] * dd1[s];
      }
      bf16x8 ah, al;
      split_bf16x8(sc, ah, al);
      const bf16x8 bg = __builtin_bit_cast(bf16x8, b);
      acc[hh] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ah, bg, acc[hh], 0, 0, 0);
      acc[hh] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(al, bg, acc[hh], 0, 0, 0);
      ks[hh] += zs;
      // dq replaces the g piece this lane read (no other lane reads it)
      *reinterpret_cast<bf16x8*>(w.g + po) = dq;
      // one head at a time: interleaving the two heads' temporaries spills
      __builtin_amdgcn_sched_barrier(0);
    }
    wave_lds_order();
  };
  auto out_line = [&](int h2) {
    return *reinterpret_cast<const u32x4*>(w.g + tile_off(t0 + 8 * h2, j));
  };
  auto out_ptr = [&](int64_t i, int h2) {
    return dQ + base + (n_lo + (sub + i * S) * kTile + t0 + 8 * h2) * row + 8 * j;
  };
  const int64_t whole = two ? (n_hi - n_lo) / kTile : 0;
  const int64_t mine_whole = whole > sub ? (whole - sub + S - 1) / S : 0;
  int64_t i0 = 0;
  for (; i0 + U <= mine_whole; i0 += U) {
#pragma unroll
    for (int u = 0; u < U; ++u) {
      stage(i0 + u, qb[u], gb[u]);
      __builtin_amdgcn_sched_barrier(0);
      issue(i0 + u + U, qb[u], gb[u]);
      __builtin_amdgcn_sched_barrier(0);
      compute(i0 + u);
      const u32x4 o0 = out_line(0), o1 = out_line(1);
      wave_lds_order();
      st16_stream(out_ptr(i0 + u, 0), o0);
      st16_stream(out_ptr(i0 + u, 1), o1);
    }
  }
  for (; i0 < mine; i0 += U) {
#pragma unroll
    for (int u = 0; u < U; ++u) {
      if (i0 + u < mine) {
        stage(i0 + u, qb[u], gb[u]);
        __builtin_amdgcn_sched_barrier(0);
        issue(i0 + u + U, qb[u], gb[u]);
        __builtin_amdgcn_sched_barrier(0);
        compute(i0 + u);
        const u32x4 o0 = out_line(0), o1 = out_line(1);
        wave_lds_order();
        const int64_t n = n_lo + (sub + (i0 + u) * S) * kTile + t0;
        if (two || j < 4) {
          if (n < n_hi) st16_stream(out_ptr(i0 + u, 0), o0);
          if (n + 8 < n_hi) st16_stream(out_ptr(i0 + u, 1), o1);
        }
      }
    }
  }
}

// bwd_kv for the pair's two heads over the tiles sub, sub + S, ... of
// [n_lo, n_hi): dk = ([dS | dz] [v | 1]^T) * [k > 0] and dv = phi(k) dS.
// slot holds the wave's k tile and v tile. Padded tokens are computed from
// row n_lo and never stored.
template <int U, int Fm, class MakeOps>
__device__ __forceinline__ void grad_kv_pair_wave(const unsigned short* __restrict__ K,
                                                  const unsigned short* __restrict__ V,
                                                  unsigned short* __restrict__ dK,
                                                  unsigned short* __restrict__ dV,
                                                  MakeOps&& make_ops, int64_t row, int64_t base,
                                                  int64_t n_lo, int64_t n_hi, int sub, int S,
                                                  bool two, unsigned char* slot) {
  const int l = lane_id();
  const int t0 = l >> 3;
  const int j = l & 7;
  const int jl = two ? j : (j & 3);
  const int g = l >> 4;
  const int col = l & 15;
  const int64_t tiles = (n_hi - n_lo + kTile - 1) / kTile;
  const int64_t mine = tiles > sub ? (tiles - sub + S - 1) / S : 0;

  u32x4 kb[U][2], vb[U][2];
  auto issue = [&](int64_t i, u32x4 (&kd)[2], u32x4 (&vd)[2]) {
    const int64_t n0 = n_lo + (sub + i * S) * kTile + t0;
#pragma unroll
    for (int h2 = 0; h2 < 2; ++h2) {
      const int64_t n = n0 + 8 * h2;
      const int64_t off = base + (n < n_hi ? n : n_lo) * row + 8 * jl;
      kd[h2] = ld16_stream(K + off);
      vd[h2] = ld16_stream(V + off);
    }
  };
#pragma unroll
  for (int u = 0; u < U; ++u) issue(u, kb[u], vb[u]);
  ApplyOperands ao[2];
  RowOperands ro[2];
  make_ops(ao, ro);

  auto compute = [&](const u32x4 (&kin)[2], const u32x4 (&vin)[2]) {
#pragma unroll
    for (int h2 = 0; h2 < 2; ++h2) {
      const int o = tile_off(t0 + 8 * h2, j);
      *reinterpret_cast<u32x4*>(slot + o) = kin[h2];
      *reinterpret_cast<u32x4*>(slot + kTileBytes + o) = vin[h2];
    }
    wave_lds_order();
#pragma unroll
    for (int hh = 0; hh < 2; ++hh) {
      const int po = tile_off(col, hh * 4 + g);
      const u32x4 kraw = *reinterpret_cast<const u32x4*>(slot + po);
      const u32x4 vraw = *reinterpret_cast<const u32x4*>(slot + kTileBytes + po);
      float y[8], x[8], dph[8];
      const u32x4 rk = relu_bf16x8(kraw);
      row_product<false>(ro[hh], __builtin_bit_cast(bf16x8, vraw), (bf16x8)0, y);
      if (Fm == kFmapRelu) {
        col_product(ao[hh], __builtin_bit_cast(bf16x8, rk), x);
      } else {
        // phi(k) in fp32, split into bf16 hi + lo: dv = hi dS + lo dS
        float pk[8], x2[8];
        widen_bf16x8(kraw, pk);
#pragma unroll
        for (int m = 0; m < 8; ++m) fmap_dfmap_hw<Fm>(pk[m], pk[m], dph[m]);
        bf16x8 hi, lo;
        split_bf16x8(pk, hi, lo);
        col_product(ao[hh], hi, x);
        col_product(ao[hh], lo, x2);
#pragma unroll
        for (int m = 0; m < 8; ++m) x[m] += x2[m];
      }
      u32x4 dk, dv;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const float d0 = y[2 * e] + ro[hh].last[2 * e];
        const float d1 = y[2 * e + 1] + ro[hh].last[2 * e + 1];
        dk[e] = Fm == kFmapRelu ? relu_gate_pk(cvt_pk_bf16(d0, d1), rk[e])
                                : cvt_pk_bf16(d0 * dph[2 * e], d1 * dph[2 * e + 1]);
        dv[e] = cvt_pk_bf16(x[2 * e], x[2 * e + 1]);
      }
      *reinterpret_cast<u32x4*>(slot + po) = dk;
      *reinterpret_cast<u32x4*>(slot + kTileBytes + po) = dv;
    }
    wave_lds_order();
  };
  auto line = [&](int tile, int h2) {
    return *reinterpret_cast<const u32x4*>(slot + tile * kTileBytes + tile_off(t0 + 8 * h2, j));
  };
  auto out_off = [&](int64_t i, int h2) {
    return base + (n_lo + (sub + i * S) * kTile + t0 + 8 * h2) * row + 8 * j;
  };
  const int64_t whole = two ? (n_hi - n_lo) / kTile : 0;
  const int64_t mine_whole = whole > sub ? (whole - sub + S - 1) / S : 0;
  int64_t i0 = 0;
  for (; i0 + U <= mine_whole; i0 += U) {
#pragma unroll
    for (int u = 0; u < U; ++u) {
      compute(kb[u], vb[u]);
      __builtin_amdgcn_sched_barrier(0);
      issue(i0 + u + U, kb[u], vb[u]);
      const u32x4 k0 = line(0, 0), k1 = line(0, 1), v0 = line(1, 0), v1 = line(1, 1);
      wave_lds_order();
      st16_stream(dK + out_off(i0 + u, 0), k0);
      st16_stream(dK + out_off(i0 + u, 1), k1);
      st16_stream(dV + out_off(i0 + u, 0), v0);
      st16_stream(dV + out_off(i0 + u, 1), v1);
    }
  }
  for (; i0 < mine; i0 += U) {
#pragma unroll
    for (int u = 0; u < U; ++u) {
      if (i0 + u < mine) {
        compute(kb[u], vb[u]);
        issue(i0 + u + U, kb[u], vb[u]);
        const u32x4 k0 = line(0, 0), k1 = line(0, 1), v0 = line(1, 0), v1 = line(1, 1);
        wave_lds_order();
        const int64_t n = n_lo + (sub + (i0 + u) * S) * kTile + t0;
        if (two || j < 4) {
          if (n < n_hi) {
            st16_stream(dK + out_off(i0 + u, 0), k0);
            st16_stream(dV + out_off(i0 + u, 0), v0);
          }
          if (n + 8 < n_hi) {
            st16_stream(dK + out_off(i0 + u, 1), k1);
            st16_stream(dV + out_off(i0 + u, 1), v1);
          }
        }
      }
    }
  }
}

// The state operands of one segment: the sum of `count` slots of the pair
// (see sum_slots_to_lds), then both heads' operands from LDS.
struct StateOps {
  const f32x4* st;
  int64_t count;
  bool two;
  f32x4* stage;
  __device__ __forceinline__ const float* sum() const {
    sum_slots_to_lds(st, count, (two ? 2 : 1) * kSF / 4, stage);
    __syncthreads();
    return reinterpret_cast<const float*>(stage);
  }
  __device__ __forceinline__ void operator()(RowOperands (&ro)[2]) const {
    const float* stf = sum();
    ro[0] = make_row_operands(stf);
    ro[1] = two ? make_row_operands(stf + kSF) : ro[0];
  }
  __device__ __forceinline__ void operator()(ApplyOperands (&ao)[2], RowOperands (&ro)[2]) const {
    const float* stf = sum();
    ao[0] = make_apply_operands(stf);
    ro[0] = make_row_operands(stf);
    ao[1] = two ? make_apply_operands(stf + kSF) : ao[0];
    ro[1] = two ? make_row_operands(stf + kSF) : ro[0];
  }
};

// bwd_q over one block's range of the flattened (unit, tile) index, on the
// state reduction's grid: one (unit, chunk) item in XCD runs when C > 0,
// else balanced ranges of Qb tiles. The forward state of a unit is the sum
// of `slot_count(unit, T, Qf)` consecutive [2][d][d+1] slots at
// src + b * sb + p * sp (pair p of batch item b): the reduction's partials
// (rule Qf), or with Qf = 0 one folded state; and the block writes its
// [dS | dz] partial of each unit it touches to grad_parts in the reduction's
// slot (the chunk, or g - first), so the partials follow the same slot rule.
template <int S, int U, int Fm = kFmapRelu>
__global__ __launch_bounds__(64 * S) void bwd_q_bf16_kernel(
    const unsigned short* __restrict__ Q, const unsigned short* __restrict__ G,
    unsigned short* __restrict__ dQ, const float* __restrict__ src, int64_t sb, int64_t sp,
    float* __restrict__ grad_parts, float eps, int64_t N, int64_t H, int64_t pairs, int64_t T,
    int64_t Qb, int64_t F, int64_t slots, int64_t Qf, int64_t C, int64_t X) {
  static_assert(2 * kWave * S >= 2 * kSF / 4, "two state elements per thread cover a pair");
  union alignas(16) Lds {
    BwdQWaveLds wave[S];
    float xchg[S][kFoldFloats][kWave];
  };
  __shared__ Lds lds;
  __shared__ f32x4 stage[2 * kSF / 4];
  const int sub = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int64_t g = blockIdx.x;
  // C > 0: (unit, chunk) items of Qb tiles in XCD runs, as the reduction's
  // chunked grid; the chunk is the slot. C = 0: balanced ranges.
  int64_t f_lo, f_hi, chunk = 0;
  if (C > 0) {
    const Item it = xcd_item(F / T, C, X);
    if (!it.valid) return;  // the whole block
    chunk = it.chunk;
    f_lo = it.unit * T + it.chunk * Qb;
    f_hi = f_lo + Qb < (it.unit + 1) * T ? f_lo + Qb : (it.unit + 1) * T;
  } else {
    f_lo = g * Qb;
    f_hi = f_lo + Qb < F ? f_lo + Qb : F;
  }
  for (int64_t unit = f_lo / T; unit * T < f_hi; ++unit) {
    const Segment sg = segment_of(unit, f_lo, f_hi, T, N, H, pairs);
    const int64_t slot = C > 0 ? chunk : g - slot_range(unit, T, Qb).first;
    const StateOps ops{reinterpret_cast<const f32x4*>(src + sg.b * sb + (sg.h >> 1) * sp),
                       slot_count(unit, T, Qf), sg.two, stage};
    f32x16 acc[2] = {(f32x16)0, (f32x16)0};
    float ks[2] = {0.0f, 0.0f};
    grad_q_pair_wave<U, Fm>(Q, G, dQ, ops, eps, H * kD, (sg.b * N * H + sg.h) * kD, sg.n_lo,
                        sg.n_hi, sub, S, sg.two, lds.wave[sub], acc, ks);
    block_sum_state<S, false>(acc, ks, lds.xchg, sub,
                              grad_parts + (unit * slots + slot) * 2 * kSF, sg.two);
    __syncthreads();  // the LDS (tiles, exchange, stage) is reused by the next segment
  }
}

// bwd_kv, one block per (unit, chunk), grouped by XCD exactly like the apply;
// a unit's [dS | dz] is the sum of bwd_q's partials (slots of grid Qr).
// (Balanced ranges of the flattened index, as in the reduction, measured
// slower: a block that straddles two units pays the state prologue twice.)
template <int S, int U, int Fm = kFmapRelu>
__global__ __launch_bounds__(64 * S) void bwd_kv_bf16_kernel(
    const unsigned short* __restrict__ K, const unsigned short* __restrict__ V,
    unsigned short* __restrict__ dK, unsigned short* __restrict__ dV,
    const float* __restrict__ grad_parts, int64_t N, int64_t H, int64_t pairs, int64_t units,
    int64_t T, int64_t C, int64_t Qa, int64_t X, int64_t Qr, int64_t slots) {
  static_assert(2 * kWave * S >= 2 * kSF / 4, "two state elements per thread cover a pair");
  __shared__ alignas(16) unsigned char tiles[S][2 * kTileBytes];
  __shared__ f32x4 stage[2 * kSF / 4];
  const int sub = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const Item it = xcd_item(units, C, X);
  if (!it.valid) return;  // the whole block
  const int64_t unit = it.unit;
  const int64_t f_lo = unit * T + it.chunk * Qa;
  const int64_t f_hi = f_lo + Qa < (unit + 1) * T ? f_lo + Qa : (unit + 1) * T;
  const Segment sg = segment_of(unit, f_lo, f_hi, T, N, H, pairs);
  const StateOps ops{reinterpret_cast<const f32x4*>(grad_parts + unit * slots * 2 * kSF),
                     slot_count(unit, T, Qr), sg.two, stage};
  grad_kv_pair_wave<U, Fm>(K, V, dK, dV, ops, H * kD, (sg.b * N * H + sg.h) * kD, sg.n_lo, sg.n_hi,
                       sub, S, sg.two, tiles[sub]);
}

// ------------------------------------------------------ causal attention
//
// Token-causal attention (query i attends to keys 0..i of its batch item),
// computed chunk-wise: an exclusive prefix of chunk states plus, inside a
// chunk, the running state and the causal terms of each 16-token tile; and
// block-causal attention with short blocks the same way. Every wave owns
// one (unit, chunk) of W consecutive tiles (the last chunk may be shorter);
// waves are numbered unit-major (wave = unit * chunks + chunk), so the 8
// waves of a block mostly stream consecutive chunks of one head pair
// (measured 1-2 us faster per kernel on the 4096px latent than 8 head pairs
// at one chunk).
//   causal_states_kernel: S_c = phi(K_c)^T [V_c | 1] per chunk, from the
//     wave's registers to parts[unit][chunk] ([2][d][d+1], both heads);
//   causal_scan_kernel: parts[unit][c] <- sum of parts[unit][0 .. c-1];
//   causal_apply_kernel: from that prefix P, tile by tile:
//     out_i = phi(q_i) (P + sum_{j <= i in the tile} phi(k_j)^T [v_j | 1])
//     split into numerator and normaliser, then P += the tile's state
//     (with blocks of 2^lg <= 16 tokens, j runs over the query's block);
//   causal_block_apply_kernel: blocks of whole tiles, block by block (see
//     there).

struct CausalWave {
  int64_t unit, chunk, b, h, n_lo, n_hi;
  bool two, valid;
};

__device__ __forceinline__ CausalWave causal_wave(int64_t units, int64_t chunks, int64_t pairs,
                                                  int64_t H, int64_t N, int64_t W, int S) {
  CausalWave c;
  const int64_t wg = blockIdx.x * (int64_t)S + __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  c.valid = wg < units * chunks;  // the grid's last block may hold spare waves
  c.unit = wg / chunks;
  c.chunk = wg - c.unit * chunks;
  c.b = c.unit / pairs;
  c.h = 2 * (c.unit - c.b * pairs);
  c.two = c.h + 1 < H;
  c.n_lo = c.chunk * W * kTile;
  c.n_hi = c.n_lo + W * kTile < N ? c.n_lo + W * kTile : N;
  return c;
}

// A head pair's state from the 32x32 MFMA accumulator layout (lane l,
// register r: row 8 (r / 4) + 4 (l / 32) + r % 4, column l % 32; ksum of
// channel c split over lanes c and c + 32) to [2][d][d+1] at dst, and back.
// store_acc_state is called by the whole wave (dst: the chunk states in the
// workspace).
__device__ __forceinline__ void store_acc_state(float* dst, const f32x16 (&acc)[2],
                                                const float (&ks)[2]) {
  const int l = lane_id();
#pragma unroll
  for (int hh = 0; hh < 2; ++hh) {
#pragma unroll
    for (int r = 0; r < 16; ++r)
      dst[hh * kSF + (8 * (r >> 2) + 4 * (l >> 5) + (r & 3)) * kSC + (l & 31)] = acc[hh][r];
    const float kq = ks[hh] + __shfl_xor(ks[hh], 32);
    if (l < 32) dst[hh * kSF + l * kSC + kD] = kq;
  }
}

__device__ __forceinline__ void load_acc_state(const float* src, f32x16 (&acc)[2],
                                               float (&ks)[2]) {
  const int l = lane_id();
#pragma unroll
  for (int hh = 0; hh < 2; ++hh) {
#pragma unroll
    for (int r = 0; r < 16; ++r)
      acc[hh][r] = src[hh * kSF + (8 * (r >> 2) + 4 * (l >> 5) + (r & 3)) * kSC + (l & 31)];
    ks[hh] = l < 32 ? src[hh * kSF + l * kSC + kD] : 0.0f;
  }
}

constexpr int kCausalStateU = 1;  // tiles a states wave issues ahead (2 measured slower)
// The states read v with ordinary loads, so that much of it is still in the
// Infinity Cache when the apply reads it again (2 x 16384 x 70 token-causal
// step 171.1 -> 157.4 us: apply 113.7 -> 99.2 us by events, states 48.3 ->
// 51.4 us). Keeping k and v both: states 56.7 us, apply as with v alone
// (161 us); k alone 160-163 us. Walking each chunk backwards made no
// difference.

template <int S>
__global__ __launch_bounds__(64 * S) void causal_states_kernel(
    const unsigned short* __restrict__ K, const unsigned short* __restrict__ V,
    float* __restrict__ parts, int64_t N, int64_t H, int64_t pairs, int64_t units,
    int64_t chunks, int64_t W) {
  __shared__ alignas(16) unsigned char slots[S][2 * kTileBytes];
  const int sub = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const CausalWave cw = causal_wave(units, chunks, pairs, H, N, W, S);
  if (!cw.valid) return;  // the whole wave; no block barrier below
  f32x16 acc[2] = {(f32x16)0, (f32x16)0};
  float ks[2] = {0.0f, 0.0f};
  reduce_pair_wave<kCausalStateU, kFmapRelu, false, true>(
      K, V, H * kD, (cw.b * N * H + cw.h) * kD, cw.n_lo, cw.n_hi, 0, 1, cw.two, slots[sub], acc,
      ks);
  store_acc_state(parts + (cw.unit * chunks + cw.chunk) * 2 * kSF, acc, ks);
}

// One thread per (unit, state element): the exclusive prefix over the
// unit's chunks, in chunk order, in place.
constexpr int kCausalScanThreads = 256;
constexpr int kCausalScanBatch = 8;
__global__ __launch_bounds__(kCausalScanThreads) void causal_scan_kernel(
    float* __restrict__ parts, int64_t units, int64_t chunks) {
  const int64_t t = blockIdx.x * (int64_t)kCausalScanThreads + threadIdx.x;
  if (t >= units * 2 * kSF) return;
  const int64_t unit = t / (2 * kSF);
  float* x = parts + unit * chunks * 2 * kSF + (t - unit * 2 * kSF);
  constexpr int kBatch = kCausalScanBatch;  // loads in flight
  float run = 0.0f;
  for (int64_t c0 = 0; c0 < chunks; c0 += kBatch) {
    float v[kBatch];
#pragma unroll
    for (int u = 0; u < kBatch; ++u) v[u] = c0 + u < chunks ? x[(c0 + u) * 2 * kSF] : 0.0f;
#pragma unroll
    for (int u = 0; u < kBatch; ++u) {
      if (c0 + u < chunks) x[(c0 + u) * 2 * kSF] = run;
      run += v[u];
    }
  }
}

// One head's 16 outputs of a tile: the state term as apply_head's, plus the
// tile's own causal term. Scores s[j][i] = phi(k_j) . phi(q_i) come from a
// 16x16x32 MFMA with phi(k) as A (row = key token, the piece at the same
// place as q's) and phi(q) as B, so a lane holds s[4 (l / 16) + r][l % 16],
// r = 0..3. Keys after the query are zeroed and the scores split into bf16
// hi + lo. One more 16x16x32 MFMA per accumulator adds [V | 1]^T s^T: its
// 32 contraction slots are, per 16-lane group g, the hi parts of keys
// 4 g .. 4 g + 3 (slots 8 g .. 8 g + 3) and their lo parts (the next four),
// so the lane's own scores are its B operand [hi | lo] and its A operand is
// v of those 4 keys at the tile row's output channel, twice (va[t], one
// transpose read); a ones operand gives the normaliser's part. Every MFMA
// on an accumulator then has one shape. (Chaining a 16x16x16 MFMA onto a
// 16x16x32 result gave results that changed by an ulp from run to run: the
// compiler left too few cycles between the two shapes, and the dependent
// MFMA sometimes read the accumulator before the lo part of the state had
// been added.) With lg > 0 a key is masked only when its block of 2^lg
// tokens comes after the query's (block-causal attention with blocks that
// divide the tile; tiles start at multiples of 16 tokens, so tile-relative
// block numbers compare like absolute ones).
__device__ __forceinline__ u32x4 causal_head(const ApplyOperands& op, u32x4 qpiece,
                                             u32x4 kpiece, s16x4 va0, s16x4 va1, float eps,
                                             int lg) {
  const bf16x8 qv = __builtin_bit_cast(bf16x8, relu_bf16x8(qpiece));
  const bf16x8 kv = __builtin_bit_cast(bf16x8, relu_bf16x8(kpiece));
  f32x4 a0 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(op.kv0_hi, qv, (f32x4)0, 0, 0, 0);
  a0 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(op.kv0_lo, qv, a0, 0, 0, 0);
  f32x4 a1 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(op.kv1_hi, qv, (f32x4)0, 0, 0, 0);
  a1 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(op.kv1_lo, qv, a1, 0, 0, 0);
  f32x4 ad = __builtin_amdgcn_mfma_f32_16x16x32_bf16(op.ks_hi, qv, (f32x4)0, 0, 0, 0);
  ad = __builtin_amdgcn_mfma_f32_16x16x32_bf16(op.ks_lo, qv, ad, 0, 0, 0);
  const f32x4 sc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kv, qv, (f32x4)0, 0, 0, 0);
  const int l = lane_id();
  const int i = l & 15, j0 = 4 * (l >> 4);
  s16x8 ss;  // [hi of the 4 scores | lo of the 4 scores]
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    const float x = (j0 + r) >> lg <= i >> lg ? sc[r] : 0.0f;
    const __bf16 h = (__bf16)x;
    ss[r] = __builtin_bit_cast(short, h);
    ss[4 + r] = __builtin_bit_cast(short, (__bf16)(x - (float)h));
  }
  const bf16x8 sb = __builtin_bit_cast(bf16x8, ss);
  const bf16x8 v0 = __builtin_bit_cast(
      bf16x8, (s16x8){va0[0], va0[1], va0[2], va0[3], va0[0], va0[1], va0[2], va0[3]});
  const bf16x8 v1 = __builtin_bit_cast(
      bf16x8, (s16x8){va1[0], va1[1], va1[2], va1[3], va1[0], va1[1], va1[2], va1[3]});
  const bf16x8 ones = __builtin_bit_cast(bf16x8, (s16x8)(short)0x3F80);  // bf16 1.0
  a0 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(v0, sb, a0, 0, 0, 0);
  a1 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(v1, sb, a1, 0, 0, 0);
  ad = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ones, sb, ad, 0, 0, 0);
  const float rinv = 1.0f / (ad[0] + eps);
  bf16x8 o;
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    o[r] = (__bf16)(a0[r] * rinv);
    o[4 + r] = (__bf16)(a1[r] * rinv);
  }
  return __builtin_bit_cast(u32x4, o);
}

// v of keys 4 (l / 16) + 0..3 at the output channel that row l % 16 of tile
// t stands for (8 (i / 4) + 4 t + i % 4, as in make_apply_operands): one
// 64-bit transpose read per lane. In each 16-lane group lane p reads token
// 4 (l / 16) + p / 4, channels 8 (p % 4) + 4 t .. + 3, and lane m receives
// element m % 4 of the rows of lanes 4 k + m / 4, k = 0..3.
__device__ __forceinline__ s16x4 gather_v_keys4(const unsigned char* vtile, int hh, int t) {
  typedef __attribute__((address_space(3))) s16x4 lds_s16x4;
  const int l = lane_id();
  const int p = l & 15;
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16(
      (lds_s16x4*)(vtile + tile_off(4 * (l >> 4) + (p >> 2), hh * 4 + (p & 3)) + 8 * t));
}

// The causal apply's running state P, kept in LDS the way its MFMAs take
// it: split into bf16 hi + lo and transposed, so the 8 contraction values a
// lane supplies (input channels 8 (l / 16) .. + 7 of the output channel its
// MFMA row stands for) are one 16-byte read. The split happens in registers
// before the store, on the values make_apply_operands would read back, so
// the operands are the same bits. Rows of kOpPitch bf16 = 80 bytes: a
// multiple of 16, and 20 banks apart, so the 32 lanes that write one
// 8-byte piece each to 32 rows meet at most two to a bank.
constexpr int kOpPitch = 40;
struct alignas(16) CausalOpsLds {  // one head at a time
  unsigned short hi[kD * kOpPitch];  // [output channel][input channel]
  unsigned short lo[kD * kOpPitch];
  unsigned short ks_hi[kD];          // [input channel]
  unsigned short ks_lo[kD];
};

// Head hh of P from the 32x32 MFMA accumulator layout (lane l holds column
// l % 32, rows 8 (r / 4) + 4 (l / 32) + r % 4: four consecutive input
// channels per quarter of acc) into ops; called by the whole wave.
__device__ __forceinline__ void store_acc_ops(CausalOpsLds& o, const f32x16& acc, float ks) {
  const int l = lane_id();
  const int col = l & 31;
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    unsigned int h[2], w[2];
#pragma unroll
    for (int e = 0; e < 2; ++e) {
      const float x0 = acc[4 * q + 2 * e], x1 = acc[4 * q + 2 * e + 1];
      h[e] = cvt_pk_bf16(x0, x1);
      w[e] = cvt_pk_bf16(x0 - __builtin_bit_cast(float, h[e] << 16),
                         x1 - __builtin_bit_cast(float, h[e] & 0xFFFF0000u));
    }
    const int at = col * kOpPitch + 8 * q + 4 * (l >> 5);
    *reinterpret_cast<u32x2*>(o.hi + at) = (u32x2){h[0], h[1]};
    *reinterpret_cast<u32x2*>(o.lo + at) = (u32x2){w[0], w[1]};
  }
  const float kq = ks + __shfl_xor(ks, 32);
  if (l < 32) {
    const __bf16 kh = (__bf16)kq;
    o.ks_hi[l] = __builtin_bit_cast(unsigned short, kh);
    o.ks_lo[l] = __builtin_bit_cast(unsigned short, (__bf16)(kq - (float)kh));
  }
}

// The apply's six A operands of the head in ops (make_apply_operands's layout).
__device__ __forceinline__ ApplyOperands load_acc_ops(const CausalOpsLds& o) {
  const int l = lane_id();
  const int g = l >> 4, i = l & 15;
  const int c0 = 8 * (i >> 2) + (i & 3);  // output channel of row i in tile 0
  const int a0 = c0 * kOpPitch + 8 * g, a1 = (c0 + 4) * kOpPitch + 8 * g;
  ApplyOperands op;
  op.kv0_hi = *reinterpret_cast<const bf16x8*>(o.hi + a0);
  op.kv0_lo = *reinterpret_cast<const bf16x8*>(o.lo + a0);
  op.kv1_hi = *reinterpret_cast<const bf16x8*>(o.hi + a1);
  op.kv1_lo = *reinterpret_cast<const bf16x8*>(o.lo + a1);
  op.ks_hi = *reinterpret_cast<const bf16x8*>(o.ks_hi + 8 * g);
  op.ks_lo = *reinterpret_cast<const bf16x8*>(o.ks_lo + 8 * g);
  return op;
}

struct alignas(16) CausalWaveLds {
  unsigned char q[kTileBytes];
  unsigned char k[kTileBytes];
  unsigned char v[kTileBytes];
  CausalOpsLds ops;
};

// Tiles whose loads an apply wave has in flight while it works on one.
constexpr int kCausalApplyU = 1;

template <int S, int U>
__global__ __launch_bounds__(64 * S) void causal_apply_kernel(
    const unsigned short* __restrict__ Q, const unsigned short* __restrict__ K,
    const unsigned short* __restrict__ V, unsigned short* __restrict__ Out,
    const float* __restrict__ parts, float eps, int64_t N, int64_t H, int64_t pairs,
    int64_t units, int64_t chunks, int64_t W, int lg) {
  __shared__ CausalWaveLds lds[S];
  const int sub = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const CausalWave cw = causal_wave(units, chunks, pairs, H, N, W, S);
  if (!cw.valid) return;  // the whole wave; no block barrier below
  CausalWaveLds& w = lds[sub];
  const int64_t row = H * kD;
  const int64_t base = (cw.b * N * H + cw.h) * kD;
  const int l = lane_id();
  const int t0 = l >> 3, j = l & 7;
  const int jl = cw.two ? j : (j & 3);
  const int g = l >> 4, col = l & 15;
  const int64_t n_lo = cw.n_lo, n_hi = cw.n_hi;
  const int64_t tiles = (n_hi - n_lo + kTile - 1) / kTile;

  f32x16 acc[2];
  float ks[2];
  load_acc_state(parts + (cw.unit * chunks + cw.chunk) * 2 * kSF, acc, ks);

  // unpredicated loads: a token past n_hi reads row n_lo (its k is zeroed
  // when staged and its output is not stored)
  u32x4 qb[U][2], kb[U][2], vb[U][2];
  auto issue = [&](int64_t i, u32x4 (&qd)[2], u32x4 (&kd)[2], u32x4 (&vd)[2]) {
#pragma unroll
    for (int h2 = 0; h2 < 2; ++h2) {
      const int64_t n = n_lo + i * kTile + t0 + 8 * h2;
      const int64_t off = base + (n < n_hi ? n : n_lo) * row + 8 * jl;
      qd[h2] = ld16_stream(Q + off);
      kd[h2] = ld16_stream(K + off);
      vd[h2] = ld16_stream(V + off);
    }
  };
  // tile i from the registers that hold it; they are refilled with tile
  // i + U as soon as the tile sits in LDS
  auto step = [&](int64_t i, u32x4 (&qd)[2], u32x4 (&kd)[2], u32x4 (&vd)[2]) {
    const int64_t n0 = n_lo + i * kTile;
#pragma unroll
    for (int h2 = 0; h2 < 2; ++h2) {
      const int o = tile_off(t0 + 8 * h2, j);
      *reinterpret_cast<u32x4*>(w.q + o) = qd[h2];
      *reinterpret_cast<u32x4*>(w.k + o) = n0 + t0 + 8 * h2 < n_hi ? kd[h2] : (u32x4)0;
      *reinterpret_cast<u32x4*>(w.v + o) = vd[h2];
    }
    wave_lds_order();
    __builtin_amdgcn_sched_barrier(0);
    issue(i + U, qd, kd, vd);
    __builtin_amdgcn_sched_barrier(0);
    u32x4 res[2];
#pragma unroll
    for (int hh = 0; hh < 2; ++hh) {
      store_acc_ops(w.ops, acc[hh], ks[hh]);  // P: every token before this tile
      wave_lds_order();
      const ApplyOperands op = load_acc_ops(w.ops);
      wave_lds_order();  // the next head's store waits for these reads
      const int po = tile_off(col, hh * 4 + g);
      const u32x4 qp = *reinterpret_cast<const u32x4*>(w.q + po);
      const u32x4 kp = *reinterpret_cast<const u32x4*>(w.k + po);
      res[hh] = causal_head(op, qp, kp, gather_v_keys4(w.v, hh, 0), gather_v_keys4(w.v, hh, 1),
                            eps, lg);
      __builtin_amdgcn_sched_barrier(0);
    }
    // P += this tile's state (keys past n_hi are zero)
#pragma unroll
    for (int hh = 0; hh < 2; ++hh) {
      const s16x8 a = gather_tokens8(w.k, hh);
      const s16x8 bv = gather_tokens8(w.v, hh);
      const s16x8 pk = __builtin_elementwise_max(a, (s16x8)0);
      acc[hh] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, pk),
                                                        __builtin_bit_cast(bf16x8, bv),
                                                        acc[hh], 0, 0, 0);
      const u32x4 wk = __builtin_bit_cast(u32x4, pk);
      float sum = 0.0f;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        sum += __builtin_bit_cast(float, wk[e] << 16);
        sum += __builtin_bit_cast(float, wk[e] & 0xFFFF0000u);
      }
      ks[hh] += sum;
    }
    wave_lds_order();
#pragma unroll
    for (int hh = 0; hh < 2; ++hh)
      *reinterpret_cast<u32x4*>(w.q + tile_off(col, hh * 4 + g)) = res[hh];
    wave_lds_order();
    const u32x4 o0 = *reinterpret_cast<const u32x4*>(w.q + tile_off(t0, j));
    const u32x4 o1 = *reinterpret_cast<const u32x4*>(w.q + tile_off(t0 + 8, j));
    wave_lds_order();
    if (cw.two || j < 4) {
      const int64_t n = n0 + t0;
      if (n < n_hi) st16_stream(Out + base + n * row + 8 * j, o0);
      if (n + 8 < n_hi) st16_stream(Out + base + (n + 8) * row + 8 * j, o1);
    }
    __builtin_amdgcn_sched_barrier(0);  // keep consecutive tiles apart (registers)
  };
#pragma unroll
  for (int u = 0; u < U; ++u) issue(u, qb[u], kb[u], vb[u]);
  // whole groups of U tiles without branches (the load counter stays exact),
  // then the rest
  int64_t i0 = 0;
  for (; i0 + U <= tiles; i0 += U) {
#pragma unroll
    for (int u = 0; u < U; ++u) step(i0 + u, qb[u], kb[u], vb[u]);
  }
#pragma unroll
  for (int u = 0; u < U; ++u)
    if (i0 + u < tiles) step(i0 + u, qb[u], kb[u], vb[u]);
}

// Block-causal attention with blocks of m >= 2 whole tiles, chunk-wise (the
// chunks are whole blocks). From its prefix P a wave walks its chunk block by
// block: first the block's k, v tiles add their states to P, then every
// query of the block reads P, which now covers exactly its own block and
// every earlier one (out = phi(q) P, the apply's arithmetic): two passes per
// block, each tensor read once, no masks. The next tile's loads (k and v in
// the first pass, q in the second, the first pass of the next block after
// the last q tile) are in flight while a tile is worked on.
template <int S>
__global__ __launch_bounds__(64 * S) void causal_block_apply_kernel(
    const unsigned short* __restrict__ Q, const unsigned short* __restrict__ K,
    const unsigned short* __restrict__ V, unsigned short* __restrict__ Out,
    const float* __restrict__ parts, float eps, int64_t N, int64_t H, int64_t pairs,
    int64_t units, int64_t chunks, int64_t W, int64_t m) {
  __shared__ CausalWaveLds lds[S];
  const int sub = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const CausalWave cw = causal_wave(units, chunks, pairs, H, N, W, S);
  if (!cw.valid) return;  // the whole wave; no block barrier below
  CausalWaveLds& w = lds[sub];
  const int64_t row = H * kD;
  const int64_t base = (cw.b * N * H + cw.h) * kD;
  const int l = lane_id();
  const int t0 = l >> 3, j = l & 7;
  const int jl = cw.two ? j : (j & 3);
  const int g = l >> 4, col = l & 15;
  const int64_t n_lo = cw.n_lo;
  // whole blocks: N is a multiple of 16 m and chunks end on block boundaries
  const int64_t blocks = (cw.n_hi - n_lo) / (m * kTile);

  f32x16 acc[2];
  float ks[2];
  load_acc_state(parts + (cw.unit * chunks + cw.chunk) * 2 * kSF, acc, ks);

  u32x4 qb[2], kb[2], vb[2];
  auto offset = [&](int64_t tile, int h2) {
    return base + (n_lo + tile * kTile + t0 + 8 * h2) * row + 8 * jl;
  };
  auto issue_kv = [&](int64_t tile) {
#pragma unroll
    for (int h2 = 0; h2 < 2; ++h2) {
      kb[h2] = ld16_stream(K + offset(tile, h2));
      vb[h2] = ld16_stream(V + offset(tile, h2));
    }
  };
  auto issue_q = [&](int64_t tile) {
#pragma unroll
    for (int h2 = 0; h2 < 2; ++h2) qb[h2] = ld16_stream(Q + offset(tile, h2));
  };
  issue_kv(0);
  for (int64_t b = 0; b < blocks; ++b) {
    const int64_t first = b * m;
    // pass 1: P += the block's k, v tiles
    for (int64_t t = 0; t < m; ++t) {
#pragma unroll
      for (int h2 = 0; h2 < 2; ++h2) {
        const int o = tile_off(t0 + 8 * h2, j);
        *reinterpret_cast<u32x4*>(w.k + o) = kb[h2];
        *reinterpret_cast<u32x4*>(w.v + o) = vb[h2];
      }
      wave_lds_order();
      __builtin_amdgcn_sched_barrier(0);
      if (t + 1 < m) {
        issue_kv(first + t + 1);
      } else {
        issue_q(first);
      }
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int hh = 0; hh < 2; ++hh) {
        const s16x8 a = gather_tokens8(w.k, hh);
        const s16x8 bv = gather_tokens8(w.v, hh);
        const s16x8 pk = __builtin_elementwise_max(a, (s16x8)0);
        acc[hh] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, pk),
                                                          __builtin_bit_cast(bf16x8, bv),
                                                          acc[hh], 0, 0, 0);
        const u32x4 wk = __builtin_bit_cast(u32x4, pk);
        float sum = 0.0f;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          sum += __builtin_bit_cast(float, wk[e] << 16);
          sum += __builtin_bit_cast(float, wk[e] & 0xFFFF0000u);
        }
        ks[hh] += sum;
      }
      wave_lds_order();
    }
    // P now covers the whole block: the apply's operands, once per block
    store_acc_ops(w.ops, acc[0], ks[0]);
    wave_lds_order();
    const ApplyOperands op0 = load_acc_ops(w.ops);
    wave_lds_order();
    store_acc_ops(w.ops, acc[1], ks[1]);
    wave_lds_order();
    const ApplyOperands op1 = load_acc_ops(w.ops);
    // pass 2: the block's queries
    for (int64_t t = 0; t < m; ++t) {
#pragma unroll
      for (int h2 = 0; h2 < 2; ++h2)
        *reinterpret_cast<u32x4*>(w.q + tile_off(t0 + 8 * h2, j)) = qb[h2];
      wave_lds_order();
      __builtin_amdgcn_sched_barrier(0);
      if (t + 1 < m) {
        issue_q(first + t + 1);
      } else if (b + 1 < blocks) {
        issue_kv(first + m);
      }
      __builtin_amdgcn_sched_barrier(0);
      const u32x4 q0 = *reinterpret_cast<const u32x4*>(w.q + tile_off(col, g));
      const u32x4 q1 = *reinterpret_cast<const u32x4*>(w.q + tile_off(col, 4 + g));
      const u32x4 r0 = apply_head(op0, q0, eps);
      const u32x4 r1 = apply_head(op1, q1, eps);
      wave_lds_order();
      *reinterpret_cast<u32x4*>(w.q + tile_off(col, g)) = r0;
      *reinterpret_cast<u32x4*>(w.q + tile_off(col, 4 + g)) = r1;
      wave_lds_order();
      const u32x4 o0 = *reinterpret_cast<const u32x4*>(w.q + tile_off(t0, j));
      const u32x4 o1 = *reinterpret_cast<const u32x4*>(w.q + tile_off(t0 + 8, j));
      wave_lds_order();
      if (cw.two || j < 4) {
        const int64_t n = n_lo + (first + t) * kTile + t0;
        st16_stream(Out + base + n * row + 8 * j, o0);
        st16_stream(Out + base + (n + 8) * row + 8 * j, o1);
      }
    }
  }
}

// ------------------------------------------------------ block-causal scan
//
// Block-causal attention runs the forward kernels on a plan whose batch
// items are the blocks (a [B][N][H][d] tensor is the same memory as
// [B * F][L][H][d] for F blocks of L tokens). Between the reduction and the
// apply, this kernel turns block states into inclusive prefix sums over the
// F blocks of each batch item. Unit u = (b * F + f) * pairs + p of that plan
// has the state sum_{j < count} src[b' * sb + p * sp + j * 2 * kSF + e]
// (b' = b * F + f; count = slot_count(u, T, Qr), 1 for a folded state).
// Thread (b, p, e) walks f = 0 .. F-1, adds block f's element e (slots in
// ascending order) to its running sum and writes the sum to
// dst[(b' * H + h) * kSF + e % kSF], the [B * F][H][d][d+1] layout the apply
// reads. Fixed order throughout, so the result is bitwise repeatable.
constexpr int kScanThreads = 256;
constexpr int kScanBlocksPerPair = (2 * kSF + kScanThreads - 1) / kScanThreads;

__global__ __launch_bounds__(kScanThreads) void scan_block_states_kernel(
    const float* __restrict__ src, int64_t sb, int64_t sp, int64_t Qr, int64_t T,
    float* __restrict__ dst, int64_t F, int64_t H, int64_t pairs) {
  const int64_t bp = blockIdx.x / kScanBlocksPerPair;  // b * pairs + p
  const int e = (blockIdx.x - bp * kScanBlocksPerPair) * kScanThreads + threadIdx.x;
  if (e >= 2 * kSF) return;
  const int64_t b = bp / pairs, p = bp - b * pairs;
  const int hh = e >= kSF ? 1 : 0;
  const int64_t h = 2 * p + hh;
  if (h >= H) return;
  float run = 0.0f;
  for (int64_t f = 0; f < F; ++f) {
    const int64_t b2 = b * F + f;
    const int64_t count = slot_count(b2 * pairs + p, T, Qr);
    const float* x = src + b2 * sb + p * sp + e;
    float sum = x[0];
    for (int64_t j = 1; j < count; ++j) sum += x[j * 2 * kSF];
    run = f == 0 ? sum : run + sum;
    dst[(b2 * H + h) * kSF + (e - hh * kSF)] = run;
  }
}

// token sub-streams per head (S) and tiles whose loads a wave issues ahead (U)
constexpr int kRedS = 8, kRedU = 2;
constexpr int kAppS = 8, kAppU = 2;
// The ELU + 1 and cos applies have more arithmetic per tile (the map, its
// hi + lo split, twice the MFMAs) and run faster with three tiles in flight
// per wave: 2 x 16384 x 70 apply, ELU + 1 65.9 -> 62.0 us, cos 63.6 -> 61.6
// us (one tile: 75.3 / 71.3 us; four: as three). ReLU's stays at two.
constexpr int kAppFmapU = 3;
template <int Fm>
constexpr int app_u() { return Fm == kFmapRelu ? kAppU : kAppFmapU; }
// Dynamic LDS the bf16 apply requests on top of its own (about 25 KB), only
// to hold it to one block (8 waves) per CU: with inputs that are not in the
// Infinity Cache, 8 streaming waves per CU move this read + write mix faster
// than 16 (measured on the 2 x 16384 x 70 forward: apply 61 -> 55 us), as
// fewer concurrent streams contend for HBM rows.
constexpr unsigned kApplyLdsPad = 64 << 10;
// Fused bf16 block shapes by head-pair units per CU (fewer bytes in flight
// per CU as more blocks share it, as for the apply): below one unit per CU,
// 8 waves with two tiles in flight each; from one, 8 waves with one tile;
// from two, 4 waves with one tile. Measured, us (256 CUs; B x N x H, units =
// B x ceil(H / 2); shape 8.2 / 8.1 / 4.1): 4 x 1024 x 70 (140 units)
// 18.3 / 20.4 / -; 8 x 1024 x 64 (256) 28.5 / 27.2 / 33.3; 8 x 1024 x 70
// (280) 36.3 / 34.0 / 36.7; 8 x 512 x 70 (280) 19.9 / 18.6 / 20.7;
// 16 x 1024 x 64 (512) 55.2 / - / 52.1; 16 x 1024 x 70 (560) 57.8 / 61.3 /
// 56.4; 16 x 512 x 70 (560) 31.1 / - / 29.2; 32 x 256 x 70 (1120) 30.6 / - /
// 30.7.
constexpr int kFusS = 8, kFusU = 2;
constexpr int kFusMidS = 8, kFusMidU = 1;
constexpr int kFusNarrowS = 4, kFusNarrowU = 1;
constexpr int kBwqS = 8, kBwqU = 1;
constexpr int kBwkvS = 8, kBwkvU = 1;
// XCDs of MI355X (the round-robin width of block dispatch). Fewer units than
// that: plain order (a unit's chunks are spread over the XCDs anyway).
constexpr int64_t kXcds = 8;
int64_t apply_xcds(const Plan& p) { return p.units >= kXcds ? kXcds : 1; }
int64_t xcd_grid(int64_t items, int64_t X) { return X * ((items + X - 1) / X); }
constexpr int kF32S = 4, kF32U = 2;

// Runs f(std::integral_constant<int, Fm>) for the feature map fmap.
template <class F>
hipError_t with_fmap(int fmap, F&& f) {
  switch (fmap) {
    case kFmapRelu: return f(std::integral_constant<int, kFmapRelu>{});
    case kFmapElu1: return f(std::integral_constant<int, kFmapElu1>{});
    case kFmapCos: return f(std::integral_constant<int, kFmapCos>{});
  }
  return hipErrorInvalidValue;
}

}  // namespace

hipError_t launch_reduce(const Plan& p, int dtype, bool fold, const void* k, const void* v,
                         float* partials, float* state, unsigned long long* ctl,
                         unsigned long long epoch, hipStream_t stream, int fmap, bool keep_k) {
  const int64_t BH = p.B * p.H;
  if (dtype != 1 && !fold) return hipErrorInvalidValue;
  return with_fmap(fmap, [&](auto fm) {
    constexpr int Fm = decltype(fm)::value;
    if (dtype == 1) {
      auto* kernel = fold      ? reduce_bf16_kernel<kRedS, kRedU, true, Fm>
                     : keep_k  ? reduce_bf16_kernel<kRedS, kRedU, false, Fm, true>
                               : reduce_bf16_kernel<kRedS, kRedU, false, Fm>;
      const bool chunked = p.red_cb > 0;
      const int64_t X = apply_xcds(p);
      const int64_t blocks = chunked ? xcd_grid(p.units * p.red_cb, X) : p.red_blocks;
      hipLaunchKernelGGL(kernel, dim3((unsigned)blocks), dim3(64 * kRedS), 0, stream,
                         static_cast<const unsigned short*>(k),
                         static_cast<const unsigned short*>(v), partials, state, ctl, epoch, p.N,
                         p.H, p.ld, p.pairs, p.tiles, chunked ? p.red_cq : p.red_q,
                         p.units * p.tiles, p.slots, chunked ? p.red_cb : int64_t(0), X);
    } else {
      hipLaunchKernelGGL((reduce_f32_kernel<kF32S, kF32U, Fm>),
                         dim3((unsigned)(p.units * p.red_chunks)), dim3(128 * kF32S), 0, stream,
                         static_cast<const float*>(k), static_cast<const float*>(v), partials,
                         state, ctl, epoch, p.N, p.H, p.ld, p.pairs, p.units, p.red_chunk,
                         p.red_chunks, BH);
    }
    return hipGetLastError();
  });
}

int block_waves(KernelKind kind, int dtype) {
  switch (kind) {
    case KernelKind::kBwdQ: return kBwqS;
    case KernelKind::kBwdKV: return kBwkvS;
    default: break;
  }
  if (dtype != 1) return 2 * kF32S;
  return kind == KernelKind::kReduce ? kRedS : kAppS;
}

int occupancy_blocks_per_cu(KernelKind kind, int dtype) {
  int n = 0;
  hipError_t e = hipErrorInvalidValue;
  switch (kind) {
    case KernelKind::kReduce:
      e = dtype == 1 ? hipOccupancyMaxActiveBlocksPerMultiprocessor(
                           &n, reduce_bf16_kernel<kRedS, kRedU, false>, 64 * kRedS, 0)
                     : hipOccupancyMaxActiveBlocksPerMultiprocessor(
                           &n, reduce_f32_kernel<kF32S, kF32U>, 128 * kF32S, 0);
      break;
    case KernelKind::kApply:
      e = dtype == 1 ? hipOccupancyMaxActiveBlocksPerMultiprocessor(
                           &n, apply_bf16_kernel<kAppS, kAppU>, 64 * kAppS, kApplyLdsPad)
                     : hipOccupancyMaxActiveBlocksPerMultiprocessor(
                           &n, apply_f32_kernel<kF32S>, 128 * kF32S, 0);
      break;
    case KernelKind::kBwdQ:
      e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, bwd_q_bf16_kernel<kBwqS, kBwqU>,
                                                       64 * kBwqS, 0);
      break;
    case KernelKind::kBwdKV:
      e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, bwd_kv_bf16_kernel<kBwkvS, kBwkvU>,
                                                       64 * kBwkvS, 0);
      break;
  }
  return e == hipSuccess && n > 0 ? n : 1;
}

// The bf16 apply's grid: (unit, chunk) items in XCD runs, or balanced ranges
// of app_q tiles when the plan says so (app_q > 0).
struct ApplyGrid {
  int64_t blocks, C, Qa, X;
};
ApplyGrid apply_grid(const Plan& p) {
  if (p.app_q > 0) return {p.app_blocks, 0, p.app_q, 1};
  const int64_t X = apply_xcds(p);
  return {xcd_grid(p.units * p.app_chunks, X), p.app_chunks, p.app_chunk / kTile, X};
}

hipError_t launch_apply(const Plan& p, int dtype, const void* q, const float* state, void* out,
                        float eps, hipStream_t stream, int fmap) {
  return with_fmap(fmap, [&](auto fm) {
    constexpr int Fm = decltype(fm)::value;
    if (dtype == 1) {
      const ApplyGrid ag = apply_grid(p);
      hipLaunchKernelGGL((apply_bf16_kernel<kAppS, app_u<Fm>(), Fm>), dim3((unsigned)ag.blocks),
                         dim3(64 * kAppS), kApplyLdsPad, stream,
                         static_cast<const unsigned short*>(q), state, p.H * kSF,
                         int64_t(2 * kSF), int64_t(0), static_cast<unsigned short*>(out), eps, p.N,
                         p.H, p.ld, p.pairs, p.units, p.tiles, ag.C, ag.Qa, ag.X);
    } else {
      hipLaunchKernelGGL((apply_f32_kernel<kF32S, Fm>), dim3((unsigned)(p.units * p.app_chunks)),
                         dim3(128 * kF32S), 0, stream, static_cast<const float*>(q), state,
                         static_cast<float*>(out), eps, p.N, p.H, p.ld, p.pairs, p.units,
                         p.app_chunk);
    }
    return hipGetLastError();
  });
}

hipError_t launch_apply_partials(const Plan& p, const void* q, const float* partials, void* out,
                                 float eps, hipStream_t stream, int fmap) {
  const int64_t sp = p.slots * 2 * kSF;
  const ApplyGrid ag = apply_grid(p);
  return with_fmap(fmap, [&](auto fm) {
    constexpr int Fm = decltype(fm)::value;
    hipLaunchKernelGGL((apply_bf16_kernel<kAppS, app_u<Fm>(), Fm>), dim3((unsigned)ag.blocks),
                       dim3(64 * kAppS), kApplyLdsPad, stream,
                       static_cast<const unsigned short*>(q), partials, p.pairs * sp, sp,
                       red_rule(p), static_cast<unsigned short*>(out), eps, p.N, p.H, p.ld,
                       p.pairs, p.units, p.tiles, ag.C, ag.Qa, ag.X);
    return hipGetLastError();
  });
}

hipError_t launch_apply_slots(const Plan& p, const void* q, const float* partials, int64_t count,
                              void* out, float eps, hipStream_t stream) {
  const int64_t sp = count * 2 * kSF;
  const ApplyGrid ag = apply_grid(p);
  hipLaunchKernelGGL((apply_bf16_kernel<kAppS, kAppU, kFmapRelu>), dim3((unsigned)ag.blocks),
                     dim3(64 * kAppS), kApplyLdsPad, stream, static_cast<const unsigned short*>(q),
                     partials, p.pairs * sp, sp, -count, static_cast<unsigned short*>(out), eps,
                     p.N, p.H, p.ld, p.pairs, p.units, p.tiles, ag.C, ag.Qa, ag.X);
  return hipGetLastError();
}

hipError_t launch_bwd_q(const Plan& p, const void* q, const void* g, void* dq,
                        const float* fwd_parts, const float* state, float* grad_parts, float eps,
                        hipStream_t stream, int fmap) {
  // the reduction's grid: (unit, chunk) items when the plan has them, else
  // balanced ranges; the [dS | dz] partials then follow the same slot rule
  const bool chunked = p.red_cb > 0;
  const int64_t X = apply_xcds(p);
  const int64_t blocks = chunked ? xcd_grid(p.units * p.red_cb, X) : p.red_blocks;
  return with_fmap(fmap, [&](auto fm) {
    constexpr int Fm = decltype(fm)::value;
    hipLaunchKernelGGL((bwd_q_bf16_kernel<kBwqS, kBwqU, Fm>), dim3((unsigned)blocks),
                       dim3(64 * kBwqS), 0, stream, static_cast<const unsigned short*>(q),
                       static_cast<const unsigned short*>(g), static_cast<unsigned short*>(dq),
                       state ? state : fwd_parts,
                       state ? p.H * kSF : p.pairs * p.slots * 2 * kSF,
                       state ? int64_t(2 * kSF) : p.slots * 2 * kSF, grad_parts, eps, p.N, p.H,
                       p.pairs, p.tiles, chunked ? p.red_cq : p.red_q, p.units * p.tiles,
                       p.slots, state ? int64_t(0) : red_rule(p),
                       chunked ? p.red_cb : int64_t(0), X);
    return hipGetLastError();
  });
}

hipError_t launch_bwd_kv(const Plan& p, const void* k, const void* v, void* dk, void* dv,
                         const float* grad_parts, hipStream_t stream, int fmap) {
  const int64_t X = apply_xcds(p);
  return with_fmap(fmap, [&](auto fm) {
    constexpr int Fm = decltype(fm)::value;
    hipLaunchKernelGGL((bwd_kv_bf16_kernel<kBwkvS, kBwkvU, Fm>),
                       dim3((unsigned)xcd_grid(p.units * p.bkv_chunks, X)),
                       dim3(64 * kBwkvS), 0, stream, static_cast<const unsigned short*>(k),
                       static_cast<const unsigned short*>(v), static_cast<unsigned short*>(dk),
                       static_cast<unsigned short*>(dv), grad_parts, p.N, p.H, p.pairs, p.units,
                       p.tiles, p.bkv_chunks, p.bkv_chunk / kTile, X, red_rule(p), p.slots);
    return hipGetLastError();
  });
}

constexpr int kCausalS = 8;  // waves per block of the causal kernels (independent waves)

hipError_t launch_causal_states(const CausalPlan& cp, const void* k, const void* v, float* parts,
                                hipStream_t stream) {
  const int64_t blocks = (cp.units * cp.chunks + kCausalS - 1) / kCausalS;
  hipLaunchKernelGGL((causal_states_kernel<kCausalS>), dim3((unsigned)blocks),
                     dim3(64 * kCausalS), 0, stream, static_cast<const unsigned short*>(k),
                     static_cast<const unsigned short*>(v), parts, cp.N, cp.H, cp.pairs,
                     cp.units, cp.chunks, cp.W);
  return hipGetLastError();
}

hipError_t launch_causal_scan(const CausalPlan& cp, float* parts, hipStream_t stream) {
  const int64_t threads = cp.units * 2 * kSF;
  hipLaunchKernelGGL(causal_scan_kernel,
                     dim3((unsigned)((threads + kCausalScanThreads - 1) / kCausalScanThreads)),
                     dim3(kCausalScanThreads), 0, stream, parts, cp.units, cp.chunks);
  return hipGetLastError();
}

hipError_t launch_causal_apply(const CausalPlan& cp, const void* q, const void* k, const void* v,
                               void* out, const float* parts, float eps, hipStream_t stream) {
  const int64_t blocks = (cp.units * cp.chunks + kCausalS - 1) / kCausalS;
  hipLaunchKernelGGL((causal_apply_kernel<kCausalS, kCausalApplyU>), dim3((unsigned)blocks),
                     dim3(64 * kCausalS), 0, stream, static_cast<const unsigned short*>(q),
                     static_cast<const unsigned short*>(k), static_cast<const unsigned short*>(v),
                     static_cast<unsigned short*>(out), parts, eps, cp.N, cp.H, cp.pairs,
                     cp.units, cp.chunks, cp.W, cp.lg);
  return hipGetLastError();
}

hipError_t launch_causal_block_apply(const CausalPlan& cp, const void* q, const void* k,
                                     const void* v, void* out, const float* parts, float eps,
                                     hipStream_t stream) {
  const int64_t blocks = (cp.units * cp.chunks + kCausalS - 1) / kCausalS;
  hipLaunchKernelGGL((causal_block_apply_kernel<kCausalS>), dim3((unsigned)blocks),
                     dim3(64 * kCausalS), 0, stream, static_cast<const unsigned short*>(q),
                     static_cast<const unsigned short*>(k), static_cast<const unsigned short*>(v),
                     static_cast<unsigned short*>(out), parts, eps, cp.N, cp.H, cp.pairs,
                     cp.units, cp.chunks, cp.W, cp.m);
  return hipGetLastError();
}

hipError_t launch_scan_blocks(const Plan& p, int dtype, int64_t F, const float* partials,
                              const float* state, float* prefix, hipStream_t stream) {
  const int64_t B = p.B / F;
  const bool bf16 = dtype == 1;
  const int64_t sb = bf16 ? p.pairs * p.slots * 2 * kSF : p.H * kSF;
  const int64_t sp = bf16 ? p.slots * 2 * kSF : int64_t(2 * kSF);
  hipLaunchKernelGGL(scan_block_states_kernel, dim3((unsigned)(B * p.pairs * kScanBlocksPerPair)),
                     dim3(kScanThreads), 0, stream, bf16 ? partials : state, sb, sp,
                     bf16 ? red_rule(p) : int64_t(0), p.tiles, prefix, F, p.H, p.pairs);
  return hipGetLastError();
}

int64_t scan_grid_threads(int64_t B, int64_t pairs) {
  return B * pairs * kScanBlocksPerPair * kScanThreads;
}

hipError_t launch_fused(const Plan& p, int dtype, int64_t cus, const void* q, const void* k,
                        const void* v, void* out, float eps, hipStream_t stream) {
  const dim3 grid((unsigned)p.units);
  if (dtype == 1) {
    const int per_cu = p.units >= 2 * cus ? 2 : p.units >= cus ? 1 : 0;
    auto* kernel = per_cu == 2   ? fused_bf16_kernel<kFusNarrowS, kFusNarrowU>
                   : per_cu == 1 ? fused_bf16_kernel<kFusMidS, kFusMidU>
                                 : fused_bf16_kernel<kFusS, kFusU>;
    const int waves = per_cu == 2 ? kFusNarrowS : per_cu == 1 ? kFusMidS : kFusS;
    hipLaunchKernelGGL(kernel, grid, dim3(64 * waves), 0, stream,
                       static_cast<const unsigned short*>(q), static_cast<const unsigned short*>(k),
                       static_cast<const unsigned short*>(v), static_cast<unsigned short*>(out),
                       eps, p.N, p.H, p.pairs);
  } else {
    hipLaunchKernelGGL((fused_f32_kernel<kF32S, kF32U>), grid, dim3(128 * kF32S), 0, stream,
                       static_cast<const float*>(q), static_cast<const float*>(k),
                       static_cast<const float*>(v), static_cast<float*>(out), eps, p.N, p.H,
                       p.pairs);
  }
  return hipGetLastError();
}

}  // namespace sana
