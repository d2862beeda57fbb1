// QKV projection with the linear-attention state in its epilogue (gfx950).
//
// The Sana review's deployment section folds linear attention's ReLU(K)^T V
// product into the QKV projection layer. Here one bf16 MFMA GEMM computes
// [q | k | v] = x W^T (x: [B][N][C] token features, W: [3D][C], the [out][in]
// layout of a linear layer; D = H d). Blocks whose output columns are Q write
// Q (bf16) to memory; blocks whose columns are one head pair's K and V never
// store them: they round the tile to bf16 (what an unfused bf16 projection
// would store), form the pair's state ReLU(K)^T [V | 1] over the tile's 256
// tokens on MFMA, and write it as one partial state. The apply of the forward
// pass then sums a head pair's partials and computes the output from Q.
//
// Tiles: 256 tokens x 128 output columns x 32 input channels per step, four
// waves per block and two blocks per CU, wave w owning tokens 64w .. 64w + 63
// of the tile (2 x 4 MFMA 32x32x16 bf16 tiles). Both operand tiles have the
// input channels contiguous (x rows and W rows), so lane l of an MFMA reads
// row l % 32 and 8 consecutive channels: one 16-byte LDS read from a tile
// stored as 64-byte rows whose 16-byte pieces are XOR-swizzled by the row.
// Each step's pieces are loaded into registers two steps ahead (two register
// sets) and stored to the other of two LDS stages between the two halves of
// the current step's MFMAs; one barrier per step.
//
// Measured on the 4096px 1.6B block (x [2, 16384, 2240]): about 1000
// TFLOP/s, 40% of the bf16 MFMA peak; the same loop with its MFMAs alone
// runs at 1620 TFLOP/s, and the fragment reads from LDS (12 per 16 MFMAs)
// account for most of the difference. Loading the stages with buffer loads
// straight to LDS (three stages, no register staging) measured the same.
#include <hip/hip_runtime.h>

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
constexpr int kBM = 256, kBN = 128, kBK = 32;
constexpr int kThreads = 256;
constexpr int kRow = kBK * 2;              // bytes per operand tile row (32 channels)
constexpr int kATile = kBM * kRow;         // 16 KB
constexpr int kBTile = kBN * kRow;         // 8 KB
constexpr int kStage = kATile + kBTile;    // 24 KB
constexpr int kKVPitch = kBM * 2 + 16;     // bytes per feature row of the transposed K|V tile
constexpr int kXchg = kBN * kKVPitch;      // exchange area after the K|V tile
// LDS: two operand stages during the loop; the epilogue reuses it for the
// transposed K|V tile and the wave exchange (the larger need, 74.5 KB), so
// two blocks fit a CU's 160 KB.
constexpr int kLds = kXchg + 2 * 17 * kWave * 4;
static_assert(2 * kStage <= kLds && kBM * kBN * 2 <= kLds, "stages and Q tile fit");
// dword 3 of a raw buffer resource on gfx950 (32-bit data format, no swizzle)
constexpr int kRsrcFlags = 0x00020000;

// Offset of 16-byte piece c (0..3) of row r in a tile of 64-byte rows: the
// piece index is XORed with (r / 4) % 4, so the 16 rows an MFMA fragment
// read touches at once (four 64-byte rows per 256-byte bank sweep) fall on
// distinct banks.
__device__ __forceinline__ int swz(int r, int c) { return (r << 6) + ((c ^ ((r >> 2) & 3)) << 4); }

struct QkvArgs {
  const unsigned short* x;  // [B][N][C]
  const unsigned short* w;  // [3D][C]
  unsigned short* q;        // [B][N][H][d]
  float* partials;          // [B][pairs][J][2][d][d+1]
  int64_t N, C, H, D, pairs;
  int64_t J;      // 256-token tiles per batch item, ceil(N / 256)
  int64_t MT;     // B * J
  int64_t nq;     // Q column tiles, ceil(D / 128)
  int64_t NT;     // nq + pairs
  int64_t GM;     // M tiles per group of the block order
  int64_t items;  // MT * NT
};

__global__ __launch_bounds__(kThreads, 2) void qkv_state_kernel(QkvArgs a) {
  __shared__ alignas(16) unsigned char lds[kLds];
  const int tid = threadIdx.x;
  const int l = tid & (kWave - 1);
  const int wv = __builtin_amdgcn_readfirstlane(tid >> 6);

  // Work item of this block: the items are cut into 8 contiguous runs, one
  // per XCD (blocks are dealt to the XCDs round robin), and ordered in groups
  // of GM M-tiles with the M-tile fastest, so the blocks an XCD runs at once
  // share a few x tiles and a few W tiles in its L2.
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
  const int64_t p = nt - a.nq;  // head pair of a K|V tile

  // Operand tiles come in through buffer loads, whose range check returns 0
  // for bytes past a resource's size: the x resource spans the tile's valid
  // tokens, so tokens past N read 0; the W tile is two resources of 64 rows
  // (Q: columns 128 nt .. +63 and +64 .. +127; K | V: the pair's 64 k rows
  // and its 64 v rows), each sized to its rows below D, so columns past D
  // (the end of Q, the missing second head of an odd pair) read 0. Offsets
  // are 32-bit within a resource (the host bounds 256 C * 2 bytes).
  const int64_t rows_a = a.N - n0 < kBM ? a.N - n0 : kBM;
  const __amdgpu_buffer_rsrc_t ra_src = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<unsigned short*>(a.x + (b * a.N + n0) * a.C), 0,
      static_cast<int>(rows_a * a.C * 2), kRsrcFlags);
  int64_t w0, w1;  // first W row of each 64-row half of the tile
  if (is_q) {
    w0 = nt * kBN;
    w1 = w0 + 64;
  } else {
    w0 = a.D + 64 * p;
    w1 = 2 * a.D + 64 * p;
  }
  const int64_t f0 = is_q ? nt * kBN : 64 * p;  // feature of the first row of each half
  auto half_rows = [&](int64_t f) { return a.D - f <= 0 ? 0 : (a.D - f < 64 ? a.D - f : 64); };
  const int64_t rows_w0 = half_rows(f0), rows_w1 = half_rows(is_q ? f0 + 64 : f0);
  const __amdgpu_buffer_rsrc_t rw_src[2] = {
      __builtin_amdgcn_make_buffer_rsrc(const_cast<unsigned short*>(a.w + w0 * a.C), 0,
                                        static_cast<int>(rows_w0 * a.C * 2), kRsrcFlags),
      __builtin_amdgcn_make_buffer_rsrc(const_cast<unsigned short*>(a.w + w1 * a.C), 0,
                                        static_cast<int>(rows_w1 * a.C * 2), kRsrcFlags)};

  // Global loads of one step: x tile 4 pieces per thread (rows lr + 64 i),
  // W tile 2 (row lr of each 64-row half), never predicated. Two register
  // sets: step j's pieces go to set j % 2 and are issued two steps before
  // they are stored to LDS, so they have two steps of multiplies to land.
  // Channels past C (a ragged last step) read the next row's; they are
  // overwritten with zeros in LDS after the store.
  const int lr = tid >> 2, lc = tid & 3;
  const int off_a = (lr * static_cast<int>(a.C) + 8 * lc) * 2;
  const int row_a = 64 * static_cast<int>(a.C) * 2;   // bytes between a thread's x rows
  u32x4 ra0[4], rb0[2], ra1[4], rb1[2];
  // A step inside C passes its channel offset as the scalar offset, so the
  // per-lane offsets are loop-invariant registers; the ragged last step adds
  // it to the lane offsets, which the range check covers.
  int vo_a[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) vo_a[i] = off_a + i * row_a;
  auto load_full = [&](int k0, u32x4 (&ra)[4], u32x4 (&rb)[2]) {
    const int kb = k0 * 2;
#pragma unroll
    for (int i = 0; i < 4; ++i)
      ra[i] = __builtin_bit_cast(
          u32x4, __builtin_amdgcn_raw_buffer_load_b128(ra_src, vo_a[i], kb, 0));
#pragma unroll
    for (int i = 0; i < 2; ++i)
      rb[i] = __builtin_bit_cast(
          u32x4, __builtin_amdgcn_raw_buffer_load_b128(rw_src[i], off_a, kb, 0));
  };
  auto load = [&](int k0, u32x4 (&ra)[4], u32x4 (&rb)[2]) {
    const int kb = k0 * 2;
#pragma unroll
    for (int i = 0; i < 4; ++i)
      ra[i] = __builtin_bit_cast(
          u32x4, __builtin_amdgcn_raw_buffer_load_b128(ra_src, vo_a[i] + kb, 0, 0));
#pragma unroll
    for (int i = 0; i < 2; ++i)
      rb[i] = __builtin_bit_cast(
          u32x4, __builtin_amdgcn_raw_buffer_load_b128(rw_src[i], off_a + kb, 0, 0));
  };
  auto store_full = [&](int s, const u32x4 (&ra)[4], const u32x4 (&rb)[2]) {
    unsigned char* A = lds + s * kStage;
    unsigned char* Bt = A + kATile;
#pragma unroll
    for (int i = 0; i < 4; ++i) *reinterpret_cast<u32x4*>(A + swz(lr + 64 * i, lc)) = ra[i];
#pragma unroll
    for (int i = 0; i < 2; ++i) *reinterpret_cast<u32x4*>(Bt + swz(lr + 64 * i, lc)) = rb[i];
  };
  auto store = [&](int s, int k0, const u32x4 (&ra)[4], const u32x4 (&rb)[2]) {
    unsigned char* A = lds + s * kStage;
    unsigned char* Bt = A + kATile;
    store_full(s, ra, rb);
    if (k0 + kBK > a.C && k0 + 8 * lc >= a.C) {  // a ragged step: this thread's pieces past C
#pragma unroll
      for (int i = 0; i < 4; ++i) *reinterpret_cast<u32x4*>(A + swz(lr + 64 * i, lc)) = (u32x4)0;
#pragma unroll
      for (int i = 0; i < 2; ++i) *reinterpret_cast<u32x4*>(Bt + swz(lr + 64 * i, lc)) = (u32x4)0;
    }
  };

  f32x16 acc[2][4];
#pragma unroll
  for (int mi = 0; mi < 2; ++mi)
#pragma unroll
    for (int ni = 0; ni < 4; ++ni) acc[mi][ni] = (f32x16)0;
  // One step's multiplies. The fragments of sub-step kk + 1 are read from
  // LDS before the MFMAs of sub-step kk are issued, so their latency hides
  // behind those MFMAs.
  // One step's multiplies: both 16-channel sub-steps' fragments are read
  // from stage s first, then the MFMAs of sub-step 0, then `between` (the
  // main loop stores the next stage there, overlapping the MFMAs), then
  // those of sub-step 1.
  auto compute_with = [&](int s, auto&& between) {
    const unsigned char* A = lds + s * kStage;
    const unsigned char* Bt = A + kATile;
    bf16x8 af[2][2], bfr[2][4];
#pragma unroll
    for (int kk = 0; kk < 2; ++kk) {
      const int c = 2 * kk + (l >> 5);
#pragma unroll
      for (int mi = 0; mi < 2; ++mi)
        af[kk][mi] = *reinterpret_cast<const bf16x8*>(A + swz(64 * wv + 32 * mi + (l & 31), c));
#pragma unroll
      for (int ni = 0; ni < 4; ++ni)
        bfr[kk][ni] = *reinterpret_cast<const bf16x8*>(Bt + swz(32 * ni + (l & 31), c));
    }
    auto mfmas = [&](int kk) {
#pragma unroll
      for (int mi = 0; mi < 2; ++mi)
#pragma unroll
        for (int ni = 0; ni < 4; ++ni)
          acc[mi][ni] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[kk][mi], bfr[kk][ni],
                                                                acc[mi][ni], 0, 0, 0);
    };
    mfmas(0);
    __builtin_amdgcn_sched_barrier(0);
    between();
    __builtin_amdgcn_sched_barrier(0);
    mfmas(1);
  };
  auto compute = [&](int s) { compute_with(s, [] {}); };

  // Steps of kBK channels (the last one ragged when C % kBK != 0). Step j
  // multiplies stage j % 2 while step j + 2's pieces load into the register
  // set step j's used; at its end step j + 1's set is stored to the other
  // stage. The loop is unrolled by two so the sets stay fixed registers.
  const int nk = static_cast<int>((a.C + kBK - 1) / kBK);
  load(0, ra0, rb0);
  if (nk > 1) load(kBK, ra1, rb1);
  store(0, 0, ra0, rb0);
  __syncthreads();
  // Main loop: steps whose loads (two ahead) and stores are whole steps
  // inside C, with nothing conditional, so the waits before the stores can
  // count exactly the loads issued after them. Then the last steps with the
  // general loads and stores.
  const int nfull = static_cast<int>(a.C / kBK);
  auto step_fast = [&](int kt, u32x4 (&ra_free)[4], u32x4 (&rb_free)[2],
                       const u32x4 (&ra_next)[4], const u32x4 (&rb_next)[2]) {
    load_full((kt + 2) * kBK, ra_free, rb_free);
    __builtin_amdgcn_sched_barrier(0);  // the loads go out before the multiplies
    // step kt + 1's pieces (loaded a step ago) are stored to the other stage
    // between the two halves of the multiplies
    compute_with(kt & 1, [&] { store_full((kt & 1) ^ 1, ra_next, rb_next); });
    __syncthreads();
  };
  auto step = [&](int kt, u32x4 (&ra_free)[4], u32x4 (&rb_free)[2], const u32x4 (&ra_next)[4],
                  const u32x4 (&rb_next)[2]) {
    const int s = kt & 1;
    if (kt + 2 < nk) load((kt + 2) * kBK, ra_free, rb_free);
    __builtin_amdgcn_sched_barrier(0);
    compute(s);
    __builtin_amdgcn_sched_barrier(0);
    if (kt + 1 < nk) store(s ^ 1, (kt + 1) * kBK, ra_next, rb_next);
    __syncthreads();
  };
  int kt = 0;
  for (; kt + 3 < nfull; kt += 2) {
    step_fast(kt, ra0, rb0, ra1, rb1);
    step_fast(kt + 1, ra1, rb1, ra0, rb0);
  }
  for (; kt < nk; kt += 2) {
    step(kt, ra0, rb0, ra1, rb1);
    if (kt + 1 < nk) step(kt + 1, ra1, rb1, ra0, rb0);
  }

  // acc[mi][ni] lane l, register r: token 64 wv + 32 mi + 8 (r / 4) + 4 (l / 32)
  // + r % 4, tile column 32 ni + l % 32.
  if (is_q) {
    // Q: bf16 to LDS token-major (256-byte rows, 16-byte pieces swizzled by
    // the token), then whole 16-byte pieces to memory
#pragma unroll
    for (int mi = 0; mi < 2; ++mi)
#pragma unroll
      for (int ni = 0; ni < 4; ++ni)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int t = 64 * wv + 32 * mi + 8 * (r >> 2) + 4 * (l >> 5) + (r & 3);
          const int f = 32 * ni + (l & 31);
          *reinterpret_cast<__bf16*>(lds + t * 256 + (((f >> 3) ^ (t & 15)) << 4) + 2 * (f & 7)) =
              (__bf16)acc[mi][ni][r];
        }
    __syncthreads();
#pragma unroll 4
    for (int i = 0; i < kBM * 16 / kThreads; ++i) {
      const int idx = tid + kThreads * i;
      const int t = idx >> 4, c = idx & 15;
      const int64_t f0 = nt * kBN + 8 * c;
      const u32x4 v = *reinterpret_cast<const u32x4*>(lds + t * 256 + ((c ^ (t & 15)) << 4));
      if (n0 + t < a.N && f0 < a.D)
        *reinterpret_cast<u32x4*>(a.q + (b * a.N + n0 + t) * a.D + f0) = v;
    }
    return;
  }

  // K | V: bf16 to LDS transposed, [tile column][token] (4 tokens, 8 bytes,
  // per write); tokens past N are written as 0, so they add nothing
#pragma unroll
  for (int mi = 0; mi < 2; ++mi)
#pragma unroll
    for (int ni = 0; ni < 4; ++ni)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int f = 32 * ni + (l & 31);
        const int t = 64 * wv + 32 * mi + 8 * g + 4 * (l >> 5);
        bf16x4 v;
#pragma unroll
        for (int e = 0; e < 4; ++e)
          v[e] = n0 + t + e < a.N ? (__bf16)acc[mi][ni][4 * g + e] : (__bf16)0.0f;
        *reinterpret_cast<bf16x4*>(lds + f * kKVPitch + 2 * t) = v;
      }
  __syncthreads();
  // The pair's state over the tile's tokens: wave w takes head w % 2 and
  // tokens 128 (w / 2) .. +127; S = ReLU(K)^T V on MFMA 32x32x16 (lane l:
  // row = K channel l % 32, column = V channel l % 32, 8 tokens 8 (l / 32)..),
  // ksum of ReLU(K) on the VALU (exact widening of bf16).
  const int hh = wv & 1, th = wv >> 1;
  f32x16 st = (f32x16)0;
  float ks = 0.0f;
#pragma unroll
  for (int s = 0; s < kBM / 2 / 16; ++s) {
    const int t0 = 128 * th + 16 * s + 8 * (l >> 5);
    s16x8 kv = *reinterpret_cast<const s16x8*>(lds + (32 * hh + (l & 31)) * kKVPitch + 2 * t0);
    const bf16x8 vv =
        *reinterpret_cast<const bf16x8*>(lds + (64 + 32 * hh + (l & 31)) * kKVPitch + 2 * t0);
    kv = __builtin_elementwise_max(kv, (s16x8)0);  // ReLU on bf16 bit patterns
    st = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, kv), vv, st, 0, 0, 0);
    const u32x4 u = __builtin_bit_cast(u32x4, kv);
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      ks += __builtin_bit_cast(float, u[e] << 16);
      ks += __builtin_bit_cast(float, u[e] & 0xFFFF0000u);
    }
  }
  float* xch = reinterpret_cast<float*>(lds + kXchg) + hh * 17 * kWave;
  if (th == 1) {
#pragma unroll
    for (int r = 0; r < 16; ++r) xch[r * kWave + l] = st[r];
    xch[16 * kWave + l] = ks;
  }
  __syncthreads();
  if (th == 0) {
#pragma unroll
    for (int r = 0; r < 16; ++r) st[r] += xch[r * kWave + l];
    ks += xch[16 * kWave + l];
    ks += __shfl_xor(ks, 32);  // lanes l and l ^ 32 hold one channel's two token halves
    float* dst = a.partials + ((b * a.pairs + p) * a.J + j) * 2 * kSF + hh * kSF;
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int i = 8 * (r >> 2) + 4 * (l >> 5) + (r & 3);
      dst[i * kSC + (l & 31)] = st[r];
    }
    if (l < 32) dst[l * kSC + kHeadDim] = ks;
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
  a.NT = a.nq + a.pairs;
  a.GM = GM;
  a.items = a.MT * a.NT;
  const int64_t grid = 8 * ((a.items + 7) / 8);
  hipLaunchKernelGGL(qkv_state_kernel, dim3((unsigned)grid), dim3(kThreads), 0, stream, a);
  return hipGetLastError();
}

int64_t qkv_grid_blocks(int64_t B, int64_t N, int64_t H) {
  const int64_t D = H * kHeadDim;
  const int64_t items = B * qkv_m_tiles(N) * ((D + kBN - 1) / kBN + (H + 1) / 2);
  return 8 * ((items + 7) / 8);
}

}  // namespace sana
