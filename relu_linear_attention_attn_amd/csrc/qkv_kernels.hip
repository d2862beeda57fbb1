// QKV projection with the linear-attention state in its epilogue (gfx950).
//
// The Sana review's deployment section folds linear attention's ReLU(K)^T V
// product into the QKV projection layer. Here one bf16 MFMA GEMM computes
// [q | k | v] = x W^T (x: [B][N][C] token features, W: [3D][C], the [out][in]
// layout of a linear layer; D = H d). Tiles whose output columns are Q write
// Q (bf16) to memory; tiles whose columns are two head pairs' K and V never
// store them: they round the tile to bf16 (what an unfused bf16 projection
// would store), form each pair's state ReLU(K)^T [V | 1] over the tile's 256
// tokens on MFMA, and write it as one partial state per pair. The apply of
// the forward pass then sums a head pair's partials and computes the output
// from Q.
//
// Tiles: 256 tokens x 256 output columns, one block of four waves per CU,
// one wave per SIMD, each owning a 128 x 128 quarter (4 x 4 MFMA 32x32x16
// bf16 tiles, accumulators in AGPRs: 0.5 fragment reads per MFMA). Operands
// come in 64-channel stages: a stage holds 128 bytes of every x and W row of
// the tile, i.e. one whole 128-byte line per row, loaded by buffer loads
// straight to LDS with 8 lanes per line. Whole lines are the point: loads of
// 64-byte half lines (32 channels per row and step) return data at about
// half the rate per CU (64 against 124..140 bytes per ns measured, with
// registers or LDS as the destination), which had held every 32-channel
// design near 1000 TFLOP/s. Two stages (128 KB); the next stage's 16 loads
// per wave are issued among the first 16 MFMAs of the current one.
//
// Epilogues from registers: Q tiles multiply W x^T, so each lane holds 4
// consecutive output columns of one token (8-byte stores); K | V tiles form
// the state from the accumulators directly (see there).
#include <hip/hip_runtime.h>

#include <type_traits>

#include "linattn_internal.h"

namespace sana {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef short s16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

constexpr int kWave = 64;
constexpr int kSC = kStateCols;    // 33
constexpr int kSF = kStateFloats;  // 1056
constexpr int kBM = 256, kBN = 256;         // tile: tokens x output columns
constexpr int kThreads = 256;
constexpr int kPair = 64;                   // channels per stage
constexpr int kPRow = kPair * 2;            // 128 bytes per row and stage
constexpr int kPA = kBM * kPRow;            // 32 KB of x rows
constexpr int kPStage = kPA + kBN * kPRow;  // 64 KB
constexpr int kLds = 2 * kPStage;           // the K | V epilogue reuses stage 0
// dword 3 of a raw buffer resource on gfx950 (32-bit data format, no
// swizzle): a load past num_records returns 0
constexpr int kRsrcFlags = 0x00020000;
constexpr int kWaitLgkm0 = 0xC07F;  // s_waitcnt lgkmcnt(0), other counters not waited

typedef __attribute__((address_space(3))) void* lds_ptr;
typedef int i32x4 __attribute__((ext_vector_type(4)));

// The four dwords of a raw buffer resource over `bytes` bytes at p, made
// wave-uniform (a load past `bytes` returns 0).
__device__ __forceinline__ i32x4 buffer_words(const void* p, int bytes) {
  const unsigned long long ad = reinterpret_cast<unsigned long long>(p);
  i32x4 r;
  r.x = __builtin_amdgcn_readfirstlane(static_cast<int>(ad & 0xFFFFFFFFu));
  r.y = __builtin_amdgcn_readfirstlane(static_cast<int>((ad >> 32) & 0xFFFFu));
  r.z = __builtin_amdgcn_readfirstlane(bytes);
  r.w = kRsrcFlags;
  return r;
}

// One 16-byte buffer load per lane straight to LDS: lane l's bytes land at
// LDS address m0 + 16 l. Written as inline assembly so that the compiler,
// which cannot tell which LDS bytes such a load writes, does not wait for
// every one in flight before each LDS read; the kernel waits (s_waitcnt
// vmcnt) for the ones it needs. Nothing lands in a register. (M0 is reserved
// to the compiler, which warns when an asm statement clobbers it; this
// file's code uses M0 nowhere else.)
#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"
__device__ __forceinline__ void load_lds16(i32x4 rsrc, int voffset, int soffset, int m0) {
  asm volatile(
      "s_mov_b32 m0, %3\n\t"
      "s_nop 0\n\t"
      "buffer_load_dwordx4 %0, %1, %2 offen lds"
      :
      : "v"(voffset), "s"(rsrc), "s"(soffset), "s"(m0)
      : "memory", "m0");
}
#pragma clang diagnostic pop

// s_waitcnt operand for "at most n vector memory operations of this wave in
// flight" (gfx9 encoding: vmcnt bits 3:0 and 15:14; expcnt and lgkmcnt at
// their maxima, i.e. not waited for).
constexpr int vm_wait(int n) { return (n & 15) | ((n >> 4) << 14) | (7 << 4) | (15 << 8); }

// Stage layout: row r (x rows 0..255, then W rows 256..511) at 128 r; its
// 16-byte piece j (channels 8 j .. 8 j + 7 of the stage) in slot
// j ^ ((r >> 1) & 7), so the 16 consecutive rows an MFMA fragment read takes
// at one piece fall on 16 distinct 16-byte bank groups.
__device__ __forceinline__ int pslot(int r, int j) { return (r << 7) + ((j ^ ((r >> 1) & 7)) << 4); }

struct QkvArgs {
  const unsigned short* x;  // [B][N][C]
  const unsigned short* w;  // [3D][C]
  unsigned short* q;        // [B][N][H][d]
  float* partials;          // [B][pairs][J][2][d][d+1]
  int64_t N, C, H, D, pairs;
  int64_t J;      // 256-token tiles per batch item, ceil(N / 256)
  int64_t MT;     // B * J
  int64_t nq;     // Q column tiles, ceil(D / 256)
  int64_t NT;     // nq + ceil(pairs / 2)
  int64_t GM;     // M tiles per group of the tile order
  int64_t items;  // MT * NT
};

__global__ __launch_bounds__(kThreads, 1) void qkv_state_kernel(QkvArgs a) {
  __shared__ alignas(16) unsigned char lds[kLds];
  const int tid = threadIdx.x;
  const int l = tid & (kWave - 1);
  const int wv = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wv & 1;   // tokens 128 wm .. +127 of the tile
  const int wn = wv >> 1;  // columns 128 wn .. +127 of the tile

  // Tile of this block: the items are cut into 8 contiguous runs, one per
  // XCD (blocks are dealt to the XCDs round robin), and ordered in groups of
  // GM token tiles with the token tile fastest, so the blocks an XCD runs at
  // once share a few x tiles and a few W tiles in its L2. Item (mt, nt):
  // token tile mt, column tile nt (Q columns 256 nt .., or K | V of head
  // pairs p0 and p0 + 1).
  constexpr int64_t X = 8;
  const int64_t per = (a.items + X - 1) / X;
  const int64_t item = (blockIdx.x % X) * per + blockIdx.x / X;
  if (item >= a.items) return;
  const int64_t group = item / (a.GM * a.NT);
  const int64_t gm = a.GM < a.MT - group * a.GM ? a.GM : a.MT - group * a.GM;
  const int64_t local = item - group * a.GM * a.NT;
  const int64_t mt = group * a.GM + local % gm;
  const int64_t nt = local / gm;
  const int64_t b = mt / a.J, j = mt - b * a.J;
  const int64_t n0 = j * kBM;
  const bool is_q = nt < a.nq;
  const int64_t p0 = 2 * (nt - a.nq);

  const int64_t rows_a = a.N - n0 < kBM ? a.N - n0 : kBM;
  const i32x4 ra_src = buffer_words(a.x + (b * a.N + n0) * a.C, static_cast<int>(rows_a * a.C * 2));
  // The B tile of a Q item is W rows 256 nt .. +255; of a K | V item,
  // [k(p0) | v(p0) | k(p0 + 1) | v(p0 + 1)], 64 rows each. Wave wv loads B
  // rows 64 wv .. +63 through a resource that ends at D (the end of Q, a
  // missing head of an odd last pair, a missing last pair), so those rows
  // read 0; the x resource ends at the tile's last valid token.
  auto half_rows = [&](int64_t f) { return a.D - f <= 0 ? 0 : (a.D - f < 64 ? a.D - f : 64); };
  i32x4 rw_src;
  {
    const int qi = wv;
    int64_t w0, f;
    if (is_q) {
      w0 = nt * kBN + 64 * qi;
      f = w0;
    } else {
      const int64_t p = p0 + (qi >> 1);
      w0 = ((qi & 1) ? 2 * a.D : a.D) + 64 * p;
      f = 64 * p;
    }
    const int64_t rows = half_rows(f);
    rw_src = buffer_words(a.w + (rows > 0 ? w0 : 0) * a.C, static_cast<int>(rows * a.C * 2));
  }
  // Stage loads straight to LDS: per wave 8 instructions for x rows
  // 64 wv + 8 i .. +7 and 8 for B rows 64 wv + 8 i .. +7; lane l lands in
  // slot l % 8 of row l / 8 and so fetches piece (l % 8) ^ ((row >> 1) & 7)
  // of that row: 8 whole 128-byte lines per instruction. Offsets are 32-bit
  // within a resource (the host bounds 256 C * 2 bytes).
  const int row_c = static_cast<int>(a.C) * 2;
  const int lrow = l >> 3, lsl = l & 7;
  int vo_a[8], vo_b[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const int ra = 64 * wv + 8 * i + lrow;   // x row in the tile
    const int rb = 8 * i + lrow;             // row in this wave's W quarter
    const int rbt = 64 * wv + rb;            // row in the B tile
    vo_a[i] = ra * row_c + ((lsl ^ ((ra >> 1) & 7)) << 4);
    vo_b[i] = rb * row_c + ((lsl ^ ((rbt >> 1) & 7)) << 4);
  }
  const int lbase = __builtin_amdgcn_readfirstlane(
      static_cast<int>(reinterpret_cast<unsigned long long>((lds_ptr)lds)));
  // load i (0..15) of stage q into LDS stage q % 2: x rows (i < 8), else B
  // rows. Inside C the channel offset goes in the scalar offset; a ragged
  // stage adds it to the lane offsets, which the range check covers.
  auto dma_one = [&](int q, int i) {
    const bool inside = q < a.C / kPair;
    const int kb = q * kPRow;
    const int so = inside ? kb : 0, vk = inside ? 0 : kb;
    const int m0 = lbase + (q & 1) * kPStage + (i < 8 ? 0 : kPA) + (64 * wv + 8 * (i & 7)) * kPRow;
    load_lds16(i < 8 ? ra_src : rw_src, (i < 8 ? vo_a[i & 7] : vo_b[i & 7]) + vk, so, m0);
  };
  auto dma_pair = [&](int q) {
#pragma unroll
    for (int i = 0; i < 16; ++i) dma_one(q, i);
  };
  // a ragged stage, once landed: its pieces at channels >= C (the next row's
  // data) are zeroed
  auto zero_tail = [&](int q) {
    unsigned char* A = lds + (q & 1) * kPStage;
    for (int idx = tid; idx < (kBM + kBN) * 8; idx += kThreads) {
      const int r = idx >> 3, j = idx & 7;
      if (q * kPair + 8 * j >= a.C)
        *reinterpret_cast<u32x4*>(A + pslot(r, j)) = (u32x4)0;  // rows >= kBM: the B tile
    }
  };

  f32x16 acc[4][4];
#pragma unroll
  for (int mi = 0; mi < 4; ++mi)
#pragma unroll
    for (int ni = 0; ni < 4; ++ni) acc[mi][ni] = (f32x16)0;
  // One stage: four 16-channel sub-steps; sub-step kk + 1's fragments are
  // read while sub-step kk's 16 MFMAs run (one read per two MFMAs). Lane l
  // of an MFMA reads row l % 32, piece 2 kk + l / 32 (8 channels). Swap:
  // D = W x^T (Q tiles), else x W^T. Pre: stage q + 1's loads go out among
  // sub-step 0's MFMAs.
  auto compute_pair = [&](int q, auto swap, auto pre) {
    constexpr bool Pre = decltype(pre)::value;
    constexpr bool Swap = decltype(swap)::value;
    const unsigned char* A = lds + (q & 1) * kPStage;
    const unsigned char* Bt = A + kPA;
    bf16x8 af[2][4], bfr[2][4];
    auto frags = [&](int kk, int buf) {
      const int j = 2 * kk + (l >> 5);
#pragma unroll
      for (int mi = 0; mi < 4; ++mi)
        af[buf][mi] = *reinterpret_cast<const bf16x8*>(A + pslot(128 * wm + 32 * mi + (l & 31), j));
#pragma unroll
      for (int ni = 0; ni < 4; ++ni)
        bfr[buf][ni] = *reinterpret_cast<const bf16x8*>(Bt + pslot(128 * wn + 32 * ni + (l & 31), j));
    };
    auto mm = [&](int buf) {
#pragma unroll
      for (int mi = 0; mi < 4; ++mi)
#pragma unroll
        for (int ni = 0; ni < 4; ++ni)
          acc[mi][ni] = Swap ? __builtin_amdgcn_mfma_f32_32x32x16_bf16(bfr[buf][ni], af[buf][mi],
                                                                       acc[mi][ni], 0, 0, 0)
                             : __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[buf][mi], bfr[buf][ni],
                                                                       acc[mi][ni], 0, 0, 0);
    };
    auto frag1 = [&](int kk, int buf, int r) {  // read r (0..7) of frags(kk, buf)
      const int jp = 2 * kk + (l >> 5);
      if (r < 4)
        af[buf][r] = *reinterpret_cast<const bf16x8*>(A + pslot(128 * wm + 32 * r + (l & 31), jp));
      else
        bfr[buf][r - 4] =
            *reinterpret_cast<const bf16x8*>(Bt + pslot(128 * wn + 32 * (r - 4) + (l & 31), jp));
    };
    frags(0, 0);
    // sub-step 0, pinned: MFMA idx, then (even idx) one of sub-step 1's
    // fragment reads, then (with the prefetch) load idx of pair q + 1
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int idx = 0; idx < 16; ++idx) {
      const int mi = idx >> 2, ni = idx & 3;
      acc[mi][ni] = Swap ? __builtin_amdgcn_mfma_f32_32x32x16_bf16(bfr[0][ni], af[0][mi],
                                                                   acc[mi][ni], 0, 0, 0)
                         : __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[0][mi], bfr[0][ni],
                                                                   acc[mi][ni], 0, 0, 0);
      if ((idx & 1) == 0) frag1(1, 1, idx >> 1);
      if (Pre) dma_one(q + 1, idx);
      __builtin_amdgcn_sched_barrier(0);
    }
#pragma unroll
    for (int kk = 1; kk < 4; ++kk) {
      __builtin_amdgcn_sched_barrier(0);
      if (kk < 3) frags(kk + 1, (kk + 1) & 1);
      mm(kk & 1);
      if (kk < 3) {
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          __builtin_amdgcn_sched_group_barrier(0x008, 2, 0);
          __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
        }
      }
    }
    __builtin_amdgcn_sched_barrier(0);
  };
  // a barrier that waits for this wave's LDS operations only (loads to LDS
  // in flight are waited for by count)
  auto barrier = [] {
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_waitcnt(kWaitLgkm0);
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
  };

  // Stages of 64 channels (the last one ragged when C % 64 != 0).
  const int np = static_cast<int>((a.C + kPair - 1) / kPair);
  const int npfull = static_cast<int>(a.C / kPair);
  dma_pair(0);
  __builtin_amdgcn_s_waitcnt(vm_wait(0));
  barrier();
  if (npfull < 1) {
    zero_tail(0);
    barrier();
  }
  // Stage q is multiplied while stage q + 1 loads into the other LDS stage;
  // then this wave waits for its loads, and one barrier frees stage q and
  // publishes everyone's stage q + 1.
  auto main_loop = [&](auto swap) {
    for (int q = 0; q + 1 < np; ++q) {
      compute_pair(q, swap, std::true_type{});
      __builtin_amdgcn_s_waitcnt(vm_wait(0));
      barrier();
      if (q + 1 >= npfull) {
        zero_tail(q + 1);
        barrier();
      }
    }
    compute_pair(np - 1, swap, std::false_type{});
    barrier();
  };
  if (is_q)
    main_loop(std::true_type{});
  else
    main_loop(std::false_type{});

  // Q blocks multiplied W x^T: acc[mi][ni] lane l, register r = 4 g + e holds
  // token 128 wm + 32 mi + l % 32, tile column 128 wn + 32 ni + 8 g + 4 (l / 32)
  // + e, so each lane stores 4 consecutive columns (8 bytes) per (mi, ni, g).
  if (is_q) {
#pragma unroll
    for (int mi = 0; mi < 4; ++mi) {
      const int64_t t = n0 + 128 * wm + 32 * mi + (l & 31);
      if (t >= a.N) continue;
      unsigned short* row = a.q + (b * a.N + t) * a.D;
#pragma unroll
      for (int ni = 0; ni < 4; ++ni)
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          const int64_t f = nt * kBN + 128 * wn + 32 * ni + 8 * g + 4 * (l >> 5);
          if (f < a.D) {
            bf16x4 v;
#pragma unroll
            for (int e = 0; e < 4; ++e) v[e] = (__bf16)acc[mi][ni][4 * g + e];
            *reinterpret_cast<bf16x4*>(row + f) = v;
          }
        }
    }
    return;
  }

  // K | V blocks (x W^T): acc[mi][ni] lane l, register r holds token
  // 128 wm + 32 mi + 8 (r / 4) + 4 (l / 32) + r % 4 and tile column
  // 128 wn + 32 ni + l % 32; columns 0..63 of the wave are k of heads 0 and 1
  // of pair p0 + wn, 64..127 their v. The state ReLU(K)^T V of head hh over
  // the wave's 128 tokens comes straight from these registers: lane l holds
  // k channel l % 32 (an MFMA A row) and v channel l % 32 (a B column) at the
  // same tokens, so registers 0..7 of both (tokens 0..15 of the 32-token
  // tile, 8 per lane half) are one 32x32x16 MFMA's operands and registers
  // 8..15 (tokens 16..31) the next. The tile is rounded to bf16 first, as a
  // bf16 projection would store it. Tokens past N hold 0 (their x rows read
  // 0), so they add nothing.
  f32x16 st[2] = {(f32x16)0, (f32x16)0};
  float ks[2] = {0.0f, 0.0f};
#pragma unroll
  for (int hh = 0; hh < 2; ++hh)
#pragma unroll
    for (int mi = 0; mi < 4; ++mi)
#pragma unroll
      for (int half = 0; half < 2; ++half) {
        s16x8 kv;
        bf16x8 vv;
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          kv[e] = __builtin_bit_cast(short, (__bf16)acc[mi][hh][8 * half + e]);
          vv[e] = (__bf16)acc[mi][2 + hh][8 * half + e];
        }
        kv = __builtin_elementwise_max(kv, (s16x8)0);  // ReLU on bf16 bit patterns
        st[hh] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, kv), vv,
                                                         st[hh], 0, 0, 0);
        const u32x4 u = __builtin_bit_cast(u32x4, kv);
#pragma unroll
        for (int e = 0; e < 4; ++e) {  // ksum: exact widening of bf16
          ks[hh] += __builtin_bit_cast(float, u[e] << 16);
          ks[hh] += __builtin_bit_cast(float, u[e] & 0xFFFF0000u);
        }
      }
  // the two token halves (waves wm = 0, 1 of a column half) are summed
  // through LDS (stage 0, free since the last barrier)
  float* xch = reinterpret_cast<float*>(lds) + wn * 2 * 17 * kWave;
  if (wm == 1) {
#pragma unroll
    for (int hh = 0; hh < 2; ++hh) {
#pragma unroll
      for (int r = 0; r < 16; ++r) xch[(hh * 17 + r) * kWave + l] = st[hh][r];
      xch[(hh * 17 + 16) * kWave + l] = ks[hh];
    }
  }
  __syncthreads();
  const int64_t p = p0 + wn;
  if (wm == 0 && p < a.pairs) {
#pragma unroll
    for (int hh = 0; hh < 2; ++hh) {
#pragma unroll
      for (int r = 0; r < 16; ++r) st[hh][r] += xch[(hh * 17 + r) * kWave + l];
      float kq = ks[hh] + xch[(hh * 17 + 16) * kWave + l];
      kq += __shfl_xor(kq, 32);  // lanes l and l ^ 32 hold one channel's two token halves
      float* dst = a.partials + ((b * a.pairs + p) * a.J + j) * 2 * kSF + hh * kSF;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int i = 8 * (r >> 2) + 4 * (l >> 5) + (r & 3);
        dst[i * kSC + (l & 31)] = st[hh][r];
      }
      if (l < 32) dst[l * kSC + kHeadDim] = kq;
    }
  }
}

}  // namespace

int64_t qkv_m_tiles(int64_t N) { return (N + kBM - 1) / kBM; }

hipError_t launch_qkv_state(const void* x, const void* w, void* q, float* partials, int64_t B,
                            int64_t N, int64_t C, int64_t H, int64_t GM, hipStream_t stream) {
  QkvArgs a;
  a.x = static_cast<const unsigned short*>(x);
  a.w = static_cast<const unsigned short*>(w);
  a.q = static_cast<unsigned short*>(q);
  a.partials = partials;
  a.N = N;
  a.C = C;
  a.H = H;
  a.D = H * kHeadDim;
  a.pairs = (H + 1) / 2;
  a.J = qkv_m_tiles(N);
  a.MT = B * a.J;
  a.nq = (a.D + kBN - 1) / kBN;
  a.NT = a.nq + (a.pairs + 1) / 2;
  a.GM = GM;
  a.items = a.MT * a.NT;
  const int64_t grid = 8 * ((a.items + 7) / 8);
  hipLaunchKernelGGL(qkv_state_kernel, dim3((unsigned)grid), dim3(kThreads), 0, stream, a);
  return hipGetLastError();
}

int64_t qkv_grid_blocks(int64_t B, int64_t N, int64_t H) {
  const int64_t D = H * kHeadDim;
  const int64_t items = B * qkv_m_tiles(N) * ((D + kBN - 1) / kBN + ((H + 1) / 2 + 1) / 2);
  return 8 * ((items + 7) / 8);
}

}  // namespace sana
