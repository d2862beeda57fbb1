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
// here ReLU runs on packed bf16 in registers, the [V | 1] padding is a second
// MFMA against a ones operand, the division is one reciprocal per token, and
// the bf16 rounding happens on the store.
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
//           transposed. ksum is the same contraction against ones.
//   apply:  out^T = KV^T phi(Q_tile)^T with v_mfma_f32_16x16x32_bf16, K = d
//           in one instruction. The fp32 state is split into bf16 hi + lo
//           parts (x = hi + lo to ~2^-17 relative), so the products keep
//           near-fp32 accuracy; phi(q) is exact in bf16. The output rows of
//           the two 16-row MFMA tiles are permuted so each lane ends up with
//           8 consecutive output channels of one token: one 16-byte store.
//           The denominator comes from a third tile whose A rows all equal
//           ksum, so it lands in the same lane and register as its numerator.
// fp32 path: plain VALU FMA kernels with the same work split (exact fp32
// products, for the fp32 contract; not the throughput path).

#include <hip/hip_runtime.h>

#include "linattn_internal.h"

namespace sana {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef short s16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

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

__device__ __forceinline__ u32x4 ld16(const void* p) {
  return *reinterpret_cast<const u32x4*>(p);
}
__device__ __forceinline__ void st16(void* p, u32x4 x) { *reinterpret_cast<u32x4*>(p) = x; }

// ReLU on 8 packed bf16: a bf16 compares like its int16 bit pattern against
// +0 (negative values and -0 have the sign bit set), so max(x, 0) as signed
// 16-bit integers is the float ReLU.
__device__ __forceinline__ u32x4 relu_bf16x8(u32x4 x) {
  s16x8 s = __builtin_bit_cast(s16x8, x);
  s = __builtin_elementwise_max(s, (s16x8)0);
  return __builtin_bit_cast(u32x4, s);
}

// ------------------------------------------------------------ bf16 reduce

constexpr int kRedRow = 64;                    // bytes of one token's head row
constexpr int kRedHalfPad = 64;                // tokens 8..15 start one half-bank-row later
constexpr int kRedTileBytes = kTile * kRedRow + kRedHalfPad;   // 1088
constexpr int kRedSlotBytes = 2 * kRedTileBytes;               // K tile + V tile

// LDS offset of token t of a staged tile. Lanes 0-31 gather token s while
// lanes 32-63 gather token 8+s; the extra 64 bytes put the two rows on
// different banks.
__device__ __forceinline__ int red_lds_off(int t) { return t * kRedRow + (t >= 8 ? kRedHalfPad : 0); }

// Accumulates phi(K)^T V and phi(K)^T 1 of one head over the tiles
// sub, sub + S, ... of the token range [n_lo, n_hi). `base` is the element
// offset of (b, n = 0, h, c = 0) and `row` the element stride between tokens.
template <int U>
__device__ __forceinline__ void reduce_bf16_wave(const unsigned short* __restrict__ K,
                                                 const unsigned short* __restrict__ V,
                                                 int64_t row, int64_t base, int64_t n_lo,
                                                 int64_t n_hi, int sub, int S,
                                                 unsigned char* slot, f32x16& acc, f32x16& accs) {
  const int l = lane_id();
  const int lt = l >> 2;           // token of the tile this lane loads
  const int lq = l & 3;            // which 16-byte quarter of the 64-byte head row
  const int wr = red_lds_off(lt) + lq * 16;
  const int rc = l & 31;           // channel this lane gathers
  const int rt = (l >> 5) * 8;     // first of the 8 tokens this lane gathers
  const int64_t tiles = (n_hi - n_lo + kTile - 1) / kTile;
  const int64_t mine = tiles > sub ? (tiles - sub + S - 1) / S : 0;

  // Loads are never predicated: a lane whose token lies outside the range
  // (ragged tail, or a tile past the end) reads row n_lo instead, which is
  // always inside the tensor, and its k is zeroed when the tile is used
  // (phi(0) = 0 removes the token from both KV and ksum). Keeping the load
  // unconditional lets the compiler keep U tiles in flight.
  u32x4 kb[U], vb[U];
  auto issue = [&](int64_t i, u32x4& kd, u32x4& vd) {
    const int64_t n = n_lo + (sub + i * S) * kTile + lt;
    const int64_t off = base + (n < n_hi ? n : n_lo) * row + lq * 8;
    kd = ld16(K + off);
    vd = ld16(V + off);
  };
#pragma unroll
  for (int u = 0; u < U; ++u) issue(u, kb[u], vb[u]);

  const bf16x8 ones = __builtin_bit_cast(bf16x8, (u32x4)0x3F803F80u);
  auto stage = [&](int64_t i, u32x4 kin, u32x4 vin) {
    const int64_t n = n_lo + (sub + i * S) * kTile + lt;
    const u32x4 kc = n < n_hi ? kin : (u32x4)0;
    *reinterpret_cast<u32x4*>(slot + wr) = kc;
    *reinterpret_cast<u32x4*>(slot + kRedTileBytes + wr) = vin;
  };
  auto consume = [&]() {
    wave_lds_order();
    s16x8 a, bv;
#pragma unroll
    for (int s = 0; s < 8; ++s) {
      const int o = red_lds_off(rt + s) + 2 * rc;
      a[s] = *reinterpret_cast<const short*>(slot + o);
      bv[s] = *reinterpret_cast<const short*>(slot + kRedTileBytes + o);
    }
    wave_lds_order();
    a = __builtin_elementwise_max(a, (s16x8)0);   // phi(k), packed
    const bf16x8 ab = __builtin_bit_cast(bf16x8, a);
    acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ab, __builtin_bit_cast(bf16x8, bv), acc, 0, 0, 0);
    accs = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ab, ones, accs, 0, 0, 0);
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
      consume();
    }
  }
#pragma unroll
  for (int u = 0; u < U; ++u) {
    if (i0 + u < mine) {
      stage(i0 + u, kb[u], vb[u]);
      consume();
    }
  }
}

// 32x32 accumulator layout: lane l, register r holds row
// 8*(r/4) + 4*(l/32) + r%4 and column l%32. Rows are k channels c, columns
// v channels j; accs holds ksum[c] in every column.
__device__ __forceinline__ void store_state_from_mfma32(float* dst, const f32x16& acc,
                                                        const f32x16& accs) {
  const int l = lane_id();
  const int j = l & 31;
  const int cb = 4 * (l >> 5);
#pragma unroll
  for (int r = 0; r < 16; ++r) {
    const int c = 8 * (r >> 2) + cb + (r & 3);
    dst[c * kSC + j] = acc[r];
    if (j == 0) dst[c * kSC + kD] = accs[r];
  }
}

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

template <int S>
struct RedShared {
  unsigned char slot[2 * S][kRedSlotBytes];
  float xchg[(S > 1 ? S - 1 : 1) * 2 * 32 * kWave];
};

// ------------------------------------------------------------- bf16 apply

struct ApplyOperands {
  bf16x8 kv0_hi, kv0_lo, kv1_hi, kv1_lo, ks_hi, ks_lo;
};

// Builds the A operands of the three 16x16x32 MFMA tiles from a [d][d+1]
// fp32 state. A lane supplies row i = l%16 and contraction indices
// k = 8*(l/16) + s, s = 0..7 (the same k the lane loads from q). Tile t row i
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

template <int U>
__device__ __forceinline__ void apply_bf16_wave(const unsigned short* __restrict__ Q,
                                                unsigned short* __restrict__ Out,
                                                const ApplyOperands& op, float eps, int64_t row,
                                                int64_t base, int64_t n_lo, int64_t n_hi, int sub,
                                                int S) {
  const int l = lane_id();
  const int g = l >> 4;
  const int col = l & 15;
  const int64_t tiles = (n_hi - n_lo + kTile - 1) / kTile;
  const int64_t mine = tiles > sub ? (tiles - sub + S - 1) / S : 0;

  // Unpredicated loads (see reduce_bf16_wave): an out-of-range token reads
  // row n_lo and its result is simply not stored.
  u32x4 qb[U];
  auto issue = [&](int64_t i, u32x4& qd) {
    const int64_t n = n_lo + (sub + i * S) * kTile + col;
    qd = ld16(Q + base + (n < n_hi ? n : n_lo) * row + 8 * g);
  };
#pragma unroll
  for (int u = 0; u < U; ++u) issue(u, qb[u]);

  auto compute = [&](u32x4 qrelu) -> u32x4 {
    const bf16x8 qv = __builtin_bit_cast(bf16x8, qrelu);
    f32x4 a0 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(op.kv0_hi, qv, (f32x4)0, 0, 0, 0);
    a0 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(op.kv0_lo, qv, a0, 0, 0, 0);
    f32x4 a1 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(op.kv1_hi, qv, (f32x4)0, 0, 0, 0);
    a1 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(op.kv1_lo, qv, a1, 0, 0, 0);
    f32x4 ad = __builtin_amdgcn_mfma_f32_16x16x32_bf16(op.ks_hi, qv, (f32x4)0, 0, 0, 0);
    ad = __builtin_amdgcn_mfma_f32_16x16x32_bf16(op.ks_lo, qv, ad, 0, 0, 0);
    const float rinv = 1.0f / (ad[0] + eps);
    bf16x8 o;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      o[r] = (__bf16)(a0[r] * rinv);
      o[4 + r] = (__bf16)(a1[r] * rinv);
    }
    return __builtin_bit_cast(u32x4, o);
  };
  auto out_ptr = [&](int64_t i) {
    return Out + base + (n_lo + (sub + i * S) * kTile + col) * row + 8 * g;
  };
  // Main loop over this wave's tiles that lie wholly inside the range: no
  // branches, unconditional stores, U loads in flight.
  const int64_t whole = (n_hi - n_lo) / kTile;
  const int64_t mine_whole = whole > sub ? (whole - sub + S - 1) / S : 0;
  int64_t i0 = 0;
  for (; i0 + U <= mine_whole; i0 += U) {
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const u32x4 qc = relu_bf16x8(qb[u]);
      // refill qb[u] only after its last use, so it keeps its registers
      __builtin_amdgcn_sched_barrier(0);
      issue(i0 + u + U, qb[u]);
      st16(out_ptr(i0 + u), compute(qc));
    }
  }
  // Remainder: fewer than U whole tiles, and possibly the ragged last tile.
#pragma unroll
  for (int u = 0; u < U; ++u) {
    if (i0 + u < mine) {
      const u32x4 o = compute(relu_bf16x8(qb[u]));
      const int64_t n = n_lo + (sub + (i0 + u) * S) * kTile + col;
      if (n < n_hi) st16(out_ptr(i0 + u), o);
    }
  }
}

// ----------------------------------------------------------- fp32 reduce

// Lane l owns state rows c = l/2, columns 16*(l%2) .. +15, and ksum[c].
template <int U>
__device__ __forceinline__ void reduce_f32_wave(const float* __restrict__ K,
                                                const float* __restrict__ V, int64_t row,
                                                int64_t base, int64_t n_lo, int64_t n_hi,
                                                int sub, int S, float* slot /*2*16*32*/,
                                                float (&acc)[17]) {
  const int l = lane_id();
  const int lt = l >> 3;        // tokens lt and lt + 8 of the tile
  const int lq = l & 7;         // 16-byte eighth of the 128-byte row
  const int c = l >> 1;
  const int jh = (l & 1) * 16;
  const int64_t tiles = (n_hi - n_lo + kTile - 1) / kTile;
  const int64_t mine = tiles > sub ? (tiles - sub + S - 1) / S : 0;

  u32x4 kb[U][2], vb[U][2];
  auto issue = [&](int64_t i, u32x4 (&kd)[2], u32x4 (&vd)[2]) {
#pragma unroll
    for (int h2 = 0; h2 < 2; ++h2) {
      const int64_t n = n_lo + (sub + i * S) * kTile + lt + 8 * h2;
      const int64_t off = base + (n < n_hi ? n : n_lo) * row + lq * 4;
      kd[h2] = ld16(K + off);
      vd[h2] = ld16(V + off);
    }
  };
#pragma unroll
  for (int u = 0; u < U; ++u) issue(u, kb[u], vb[u]);

  float* ks = slot;
  float* vs = slot + kTile * kD;
  for (int64_t i0 = 0; i0 < mine; i0 += U) {
#pragma unroll
    for (int u = 0; u < U; ++u) {
      if (i0 + u < mine) {
#pragma unroll
        for (int h2 = 0; h2 < 2; ++h2) {
          const int64_t n = n_lo + (sub + (i0 + u) * S) * kTile + lt + 8 * h2;
          st16(ks + (lt + 8 * h2) * kD + lq * 4, n < n_hi ? kb[u][h2] : (u32x4)0);
          st16(vs + (lt + 8 * h2) * kD + lq * 4, vb[u][h2]);
        }
        issue(i0 + u + U, kb[u], vb[u]);
        wave_lds_order();
#pragma unroll 4
        for (int t = 0; t < kTile; ++t) {
          const float kc = fmaxf(ks[t * kD + c], 0.0f);
#pragma unroll
          for (int m = 0; m < 16; ++m) acc[m] = __builtin_fmaf(kc, vs[t * kD + jh + m], acc[m]);
          acc[16] += kc;
        }
        wave_lds_order();
      }
    }
  }
}

__device__ __forceinline__ void store_state_from_f32(float* dst, const float (&acc)[17]) {
  const int l = lane_id();
  const int c = l >> 1;
  const int jh = (l & 1) * 16;
#pragma unroll
  for (int m = 0; m < 16; ++m) dst[c * kSC + jh + m] = acc[m];
  if (jh == 0) dst[c * kSC + kD] = acc[16];
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

// Lane l computes token n_lo + 64*tile + l of one head.
__device__ __forceinline__ void apply_f32_wave(const float* __restrict__ Q, float* __restrict__ Out,
                                               const float* stp /*padded LDS*/, float eps,
                                               int64_t row, int64_t base, int64_t n_lo,
                                               int64_t n_hi, int sub, int S) {
  const int l = lane_id();
  const int64_t tiles = (n_hi - n_lo + kWave - 1) / kWave;
  for (int64_t t = sub; t < tiles; t += S) {
    const int64_t n = n_lo + t * kWave + l;
    if (n >= n_hi) continue;
    const float* qp = Q + base + n * row;
    float q[kD];
#pragma unroll
    for (int c4 = 0; c4 < kD / 4; ++c4) {
      // bit-cast whole vectors only: a bit-cast of one vector element is
      // mis-lowered by this compiler (it reads element 0)
      const f32x4 x = __builtin_bit_cast(f32x4, ld16(qp + 4 * c4));
#pragma unroll
      for (int e = 0; e < 4; ++e) q[4 * c4 + e] = fmaxf(x[e], 0.0f);
    }
    float num[kD + 1];
#pragma unroll
    for (int j = 0; j <= kD; ++j) num[j] = 0.0f;
#pragma unroll
    for (int c = 0; c < kD; ++c) {
      const float qc = q[c];
      const float* sr = stp + c * kPadCols;
#pragma unroll
      for (int j4 = 0; j4 < 9; ++j4) {
        const f32x4 s4 = *reinterpret_cast<const f32x4*>(sr + 4 * j4);
#pragma unroll
        for (int e = 0; e < 4; ++e)
          if (4 * j4 + e <= kD) num[4 * j4 + e] = __builtin_fmaf(qc, s4[e], num[4 * j4 + e]);
      }
    }
    const float rinv = 1.0f / (num[kD] + eps);
    float* op = Out + base + n * row;
#pragma unroll
    for (int c4 = 0; c4 < kD / 4; ++c4) {
      f32x4 o;
#pragma unroll
      for (int e = 0; e < 4; ++e) o[e] = num[4 * c4 + e] * rinv;
      st16(op + 4 * c4, __builtin_bit_cast(u32x4, o));
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

template <int S, int U>
__global__ __launch_bounds__(128 * S) void reduce_bf16_kernel(
    const unsigned short* __restrict__ K, const unsigned short* __restrict__ V,
    float* __restrict__ partials, int64_t N, int64_t H, int64_t pairs, int64_t units,
    int64_t chunk, int64_t BH) {
  __shared__ RedShared<S> sh;
  const BlockCoords bc = block_coords(pairs, units, H);
  const int64_t n_lo = bc.p * chunk;
  const int64_t n_hi = n_lo + chunk < N ? n_lo + chunk : N;
  f32x16 acc = (f32x16)0, accs = (f32x16)0;
  if (bc.active)
    reduce_bf16_wave<U>(K, V, H * kD, (bc.b * N * H + bc.h) * kD, n_lo, n_hi, bc.sub, S,
                        sh.slot[threadIdx.x >> 6], acc, accs);
  float regs[32];
#pragma unroll
  for (int r = 0; r < 16; ++r) {
    regs[r] = acc[r];
    regs[16 + r] = accs[r];
  }
  combine_substreams<S, 32>(regs, sh.xchg, bc.hh, bc.sub);
#pragma unroll
  for (int r = 0; r < 16; ++r) {
    acc[r] = regs[r];
    accs[r] = regs[16 + r];
  }
  if (bc.active && bc.sub == 0)
    store_state_from_mfma32(partials + (bc.p * BH + bc.b * H + bc.h) * kSF, acc, accs);
}

template <int S, int U>
__global__ __launch_bounds__(128 * S) void reduce_f32_kernel(
    const float* __restrict__ K, const float* __restrict__ V, float* __restrict__ partials,
    int64_t N, int64_t H, int64_t pairs, int64_t units, int64_t chunk, int64_t BH) {
  __shared__ float slot[2 * S][2 * kTile * kD];
  __shared__ float xchg[(S > 1 ? S - 1 : 1) * 2 * 17 * kWave];
  const BlockCoords bc = block_coords(pairs, units, H);
  const int64_t n_lo = bc.p * chunk;
  const int64_t n_hi = n_lo + chunk < N ? n_lo + chunk : N;
  float acc[17];
#pragma unroll
  for (int r = 0; r < 17; ++r) acc[r] = 0.0f;
  if (bc.active)
    reduce_f32_wave<U>(K, V, H * kD, (bc.b * N * H + bc.h) * kD, n_lo, n_hi, bc.sub, S,
                       slot[threadIdx.x >> 6], acc);
  combine_substreams<S, 17>(acc, xchg, bc.hh, bc.sub);
  if (bc.active && bc.sub == 0)
    store_state_from_f32(partials + (bc.p * BH + bc.b * H + bc.h) * kSF, acc);
}

// state[e] = sum_{p < P} partials[p][e], p ascending.
__global__ __launch_bounds__(256) void combine_kernel(const float* __restrict__ partials,
                                                      float* __restrict__ state, int64_t total,
                                                      int64_t P) {
  const int64_t e = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (e >= total) return;
  float s = partials[e];
  for (int64_t p = 1; p < P; ++p) s += partials[p * total + e];
  state[e] = s;
}

template <int S, int U>
__global__ __launch_bounds__(128 * S) void apply_bf16_kernel(
    const unsigned short* __restrict__ Q, const float* __restrict__ state,
    unsigned short* __restrict__ Out, float eps, int64_t N, int64_t H, int64_t pairs,
    int64_t units, int64_t chunk) {
  const BlockCoords bc = block_coords(pairs, units, H);
  if (!bc.active) return;
  const int64_t n_lo = bc.p * chunk;
  const int64_t n_hi = n_lo + chunk < N ? n_lo + chunk : N;
  const ApplyOperands op = make_apply_operands(state + (bc.b * H + bc.h) * kSF);
  apply_bf16_wave<U>(Q, Out, op, eps, H * kD, (bc.b * N * H + bc.h) * kD, n_lo, n_hi, bc.sub, S);
}

template <int S>
__global__ __launch_bounds__(128 * S) void apply_f32_kernel(
    const float* __restrict__ Q, const float* __restrict__ state, float* __restrict__ Out,
    float eps, int64_t N, int64_t H, int64_t pairs, int64_t units, int64_t chunk) {
  __shared__ float stp[2][kD * kPadCols];
  const BlockCoords bc = block_coords(pairs, units, H);
  if (bc.active && bc.sub == 0) stage_state_padded(stp[bc.hh], state + (bc.b * H + bc.h) * kSF);
  __syncthreads();
  if (!bc.active) return;
  const int64_t n_lo = bc.p * chunk;
  const int64_t n_hi = n_lo + chunk < N ? n_lo + chunk : N;
  apply_f32_wave(Q, Out, stp[bc.hh], eps, H * kD, (bc.b * N * H + bc.h) * kD, n_lo, n_hi, bc.sub, S);
}

// One block per (b, head pair) over all N tokens: reduce into registers,
// combine sub-streams through LDS, keep the state in LDS, apply.
template <int S, int U>
__global__ __launch_bounds__(128 * S) void fused_bf16_kernel(
    const unsigned short* __restrict__ Q, const unsigned short* __restrict__ K,
    const unsigned short* __restrict__ V, unsigned short* __restrict__ Out, float eps,
    int64_t N, int64_t H, int64_t pairs) {
  __shared__ RedShared<S> sh;
  __shared__ float st[2][kSF];
  const BlockCoords bc = block_coords(pairs, (int64_t)gridDim.x, H);
  const int64_t base = (bc.b * N * H + bc.h) * kD;
  f32x16 acc = (f32x16)0, accs = (f32x16)0;
  if (bc.active)
    reduce_bf16_wave<U>(K, V, H * kD, base, 0, N, bc.sub, S, sh.slot[threadIdx.x >> 6], acc, accs);
  float regs[32];
#pragma unroll
  for (int r = 0; r < 16; ++r) {
    regs[r] = acc[r];
    regs[16 + r] = accs[r];
  }
  combine_substreams<S, 32>(regs, sh.xchg, bc.hh, bc.sub);
  if (bc.active && bc.sub == 0) {
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      acc[r] = regs[r];
      accs[r] = regs[16 + r];
    }
    store_state_from_mfma32(st[bc.hh], acc, accs);
  }
  __syncthreads();
  if (!bc.active) return;
  const ApplyOperands op = make_apply_operands(st[bc.hh]);
  apply_bf16_wave<U>(Q, Out, op, eps, H * kD, base, 0, N, bc.sub, S);
}

template <int S, int U>
__global__ __launch_bounds__(128 * S) void fused_f32_kernel(
    const float* __restrict__ Q, const float* __restrict__ K, const float* __restrict__ V,
    float* __restrict__ Out, float eps, int64_t N, int64_t H, int64_t pairs) {
  __shared__ float slot[2 * S][2 * kTile * kD];
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
  if (bc.active && bc.sub == 0) store_state_from_f32(st[bc.hh], acc);
  __syncthreads();
  if (bc.active && bc.sub == 0) stage_state_padded(stp[bc.hh], st[bc.hh]);
  __syncthreads();
  if (!bc.active) return;
  apply_f32_wave(Q, Out, stp[bc.hh], eps, H * kD, base, 0, N, bc.sub, S);
}

constexpr int kRedS = 2, kRedU = 4;
constexpr int kAppS = 2, kAppU = 4;
constexpr int kFusS = 4, kFusU = 2;
constexpr int kF32S = 2, kF32U = 2;

}  // namespace

hipError_t launch_reduce(const Plan& p, int dtype, const void* k, const void* v, float* partials,
                         hipStream_t stream) {
  const dim3 grid((unsigned)(p.units * p.red_chunks));
  const int64_t BH = p.B * p.H;
  if (dtype == 1) {
    hipLaunchKernelGGL((reduce_bf16_kernel<kRedS, kRedU>), grid, dim3(128 * kRedS), 0, stream,
                       static_cast<const unsigned short*>(k), static_cast<const unsigned short*>(v),
                       partials, p.N, p.H, p.pairs, p.units, p.red_chunk, BH);
  } else {
    hipLaunchKernelGGL((reduce_f32_kernel<kF32S, kF32U>), grid, dim3(128 * kF32S), 0, stream,
                       static_cast<const float*>(k), static_cast<const float*>(v), partials, p.N,
                       p.H, p.pairs, p.units, p.red_chunk, BH);
  }
  return hipGetLastError();
}

hipError_t launch_combine(const Plan& p, const float* partials, float* state, hipStream_t stream) {
  const int64_t total = p.B * p.H * kStateFloats;
  const dim3 grid((unsigned)((total + 255) / 256));
  hipLaunchKernelGGL(combine_kernel, grid, dim3(256), 0, stream, partials, state, total,
                     p.red_chunks);
  return hipGetLastError();
}

hipError_t launch_apply(const Plan& p, int dtype, const void* q, const float* state, void* out,
                        float eps, hipStream_t stream) {
  const dim3 grid((unsigned)(p.units * p.app_chunks));
  if (dtype == 1) {
    hipLaunchKernelGGL((apply_bf16_kernel<kAppS, kAppU>), grid, dim3(128 * kAppS), 0, stream,
                       static_cast<const unsigned short*>(q), state,
                       static_cast<unsigned short*>(out), eps, p.N, p.H, p.pairs, p.units,
                       p.app_chunk);
  } else {
    hipLaunchKernelGGL((apply_f32_kernel<kF32S>), grid, dim3(128 * kF32S), 0, stream,
                       static_cast<const float*>(q), state, static_cast<float*>(out), eps, p.N,
                       p.H, p.pairs, p.units, p.app_chunk);
  }
  return hipGetLastError();
}

hipError_t launch_fused(const Plan& p, int dtype, const void* q, const void* k, const void* v,
                        void* out, float eps, hipStream_t stream) {
  const dim3 grid((unsigned)p.units);
  if (dtype == 1) {
    hipLaunchKernelGGL((fused_bf16_kernel<kFusS, kFusU>), grid, dim3(128 * kFusS), 0, stream,
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
