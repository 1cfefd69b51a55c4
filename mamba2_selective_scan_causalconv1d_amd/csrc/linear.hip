// The projections around the mixer path for gfx950: dst[M, N] = x[M, K] . w[N, K]^T in
// bf16 with fp32 accumulation (the layout of a linear layer's weight, one row per output
// feature), one rounding to bf16.  in_proj produces the z, xBC and dt columns (three calls
// on row slices of one weight), out_proj maps the norm's output back to the model width.
//
// Two kernels: 256 x 256 tiles with direct-to-LDS copies (below) where M, N >= 256 and K is
// a multiple of 64 (the layer's shapes), and 128 x 128 tiles for every other shape.
//
// 128 x 128 tiling: a 256-thread workgroup computes a 128 x 128 block of dst, each wavefront a
// 64 x 64 quarter as 4 x 4 tiles of v_mfma_f32_16x16x32_bf16.  K advances 64 at a time:
// the x and w rows of the step (16 KiB each) are loaded into registers two steps ahead
// (two register sets, 64 KiB in flight per workgroup), written to a double-buffered LDS
// tile (rows padded to 144 bytes, so the 16 rows a fragment read touches fall in distinct
// bank groups) and read back as MFMA fragments
// (lane l: row l % 16, k 8 (l / 16) .. +7), one barrier per step.  The product is formed
// as (w x^T)^T: a lane then holds 4 consecutive output columns of one row, stored as 8
// bytes.  Rows and k past the matrix edges are loaded from a clamped address and zeroed
// when written to LDS.
//
// Workgroup -> tile: consecutive workgroups go to different XCDs (each with its own L2),
// so the tiles are dealt XCD by XCD in row-block order: the workgroups resident on one XCD
// share the x rows of the same few row blocks, which its L2 then fetches once.
#include "common.h"

namespace m2 {
namespace {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr int BM = 128, BN = 128, BK = 64;
constexpr int LDR = BK + 8;  // bf16 elements per LDS row (144 bytes)
constexpr int kXcds = 8;

__device__ __forceinline__ f32x4 mfma(const u32x4& a, const u32x4& b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, a), __builtin_bit_cast(bf16x8_t, b),
                                                  c, 0, 0, 0);
}

__global__ __launch_bounds__(256, 2) void linear_bf16_kernel(bf16_t* __restrict__ dst, const bf16_t* __restrict__ x,
                                                             const bf16_t* __restrict__ w, int M, int N, int K,
                                                             int tiles_n, int remap) {
  __shared__ __attribute__((aligned(16))) bf16_t sA[2][BM * LDR];
  __shared__ __attribute__((aligned(16))) bf16_t sB[2][BN * LDR];
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1;

  int t = blockIdx.x;
  if (remap) {  // the tiles of XCD x are the x-th contiguous share of the row-major tile order
    const int per = gridDim.x / kXcds;
    t = (blockIdx.x % kXcds) * per + blockIdx.x / kXcds;
  }
  const int m0 = (t / tiles_n) * BM;
  const int n0 = (t % tiles_n) * BN;

  // global -> register staging: unit i = tid + 256 j is row i / 8, k 8 (i % 8) of the step.
  // Steps past the end load the last step again (clamped, unconditional, so every step issues
  // the same loads and the compiler's waits stay exact) and are never stored.
  const int nk = (K + BK - 1) / BK;
  // loads from clamped (always valid) addresses; the units past the edges are zeroed where
  // the registers are written to LDS, so no load result is needed before then
  auto gload = [&](u32x4* ra, u32x4* rb, int kt) {
    const int k0 = min(kt, nk - 1) * BK;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int i = tid + 256 * j;
      const int row = i >> 3;
      const int kc = min(k0 + 8 * (i & 7), K - 8);
      // 32-bit element offsets (M K, N K < 2^31): a uniform base plus a 32-bit lane offset
      const uint32_t oa = (uint32_t)min(m0 + row, M - 1) * (uint32_t)K + (uint32_t)kc;
      const uint32_t ob = (uint32_t)min(n0 + row, N - 1) * (uint32_t)K + (uint32_t)kc;
      ra[j] = *reinterpret_cast<const u32x4*>(x + oa);
      rb[j] = *reinterpret_cast<const u32x4*>(w + ob);
    }
  };
  auto lstore = [&](const u32x4* ra, const u32x4* rb, int kt, int buf) {
    const u32x4 z = {0u, 0u, 0u, 0u};
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int i = tid + 256 * j;
      const int row = i >> 3;
      const bool kin = kt * BK + 8 * (i & 7) < K;
      const int off = row * LDR + 8 * (i & 7);
      *reinterpret_cast<u32x4*>(&sA[buf][off]) = (kin && m0 + row < M) ? ra[j] : z;
      *reinterpret_cast<u32x4*>(&sB[buf][off]) = (kin && n0 + row < N) ? rb[j] : z;
    }
  };

  f32x4 acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

  const int frow = lane & 15, fk = 8 * (lane >> 4);
  auto compute = [&](int buf) {
#pragma unroll
    for (int kk = 0; kk < 2; ++kk) {
      u32x4 af[4], bf[4];
#pragma unroll
      for (int i = 0; i < 4; ++i)
        af[i] = *reinterpret_cast<const u32x4*>(&sA[buf][(wm * 64 + 16 * i + frow) * LDR + 32 * kk + fk]);
#pragma unroll
      for (int j = 0; j < 4; ++j)
        bf[j] = *reinterpret_cast<const u32x4*>(&sB[buf][(wn * 64 + 16 * j + frow) * LDR + 32 * kk + fk]);
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = mfma(bf[j], af[i], acc[i][j]);
    }
  };

  // Two steps of loads in flight: registers 0 and 1 alternate, each filled two steps ahead.
  u32x4 ra0[4], rb0[4], ra1[4], rb1[4];
  gload(ra0, rb0, 0);
  gload(ra1, rb1, 1);
  lstore(ra0, rb0, 0, 0);
  __syncthreads();
  for (int kt = 0; kt < nk; kt += 2) {
    gload(ra0, rb0, kt + 2);
    compute(0);
    if (kt + 1 < nk) lstore(ra1, rb1, kt + 1, 1);
    __syncthreads();
    if (kt + 1 >= nk) break;
    gload(ra1, rb1, kt + 3);
    compute(1);
    if (kt + 2 < nk) lstore(ra0, rb0, kt + 2, 0);
    __syncthreads();
  }

  // lane l holds dst[row l % 16 of the tile][columns 4 (l / 16) .. +3]
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int m = m0 + wm * 64 + 16 * i + frow;
    if (m >= M) continue;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int n = n0 + wn * 64 + 16 * j + 4 * (lane >> 4);
      if (n < N) {
        const f32x4 o = acc[i][j];
        *reinterpret_cast<uint2*>(dst + (size_t)m * N + n) = make_uint2(pack_bf16x2(o[0], o[1]), pack_bf16x2(o[2], o[3]));
      }
    }
  }
}

// ---------------------------------------------------------------- large tiles
//
// For M, N >= 256 and K a multiple of 64: a 512-thread workgroup computes a 256 x 256 block of
// dst, wavefront (wm, wn) a 128 x 64 part of it (8 x 4 MFMA tiles, 128 accumulators per lane).
// K advances 64 at a time through two LDS stages of 64 KiB (the step's 256 x rows and 256 w
// rows, 128 bytes each): the copies of step k + 1 are issued when step k starts, one barrier
// per step.  The copies are buffer loads that write LDS directly (no registers, no LDS
// stores): each instruction fills 1 KiB, 8 rows of 8 units of 16 bytes, so every lane group
// fetches a whole 128-byte line, and each lane fetches the global unit that lands in its slot.
// Unit u of tile row r sits in slot u ^ s(r % 16), s chosen so that the 16 rows a fragment
// read touches fall in distinct bank groups.  Rows past M or N read as zero (out-of-range
// buffer offsets).  The result leaves through LDS: each wavefront writes its bf16 values into
// the tile, then every row is stored as full 512-byte runs, 16 bytes per lane (8-byte stores
// straight from the accumulators, a quarter line each, were measured 5-20 % slower).

constexpr int LBM = 256, LBN = 256, LBK = 64, LNS = 2;

#define M2_LDS_AS __attribute__((address_space(3)))
typedef uint32_t u32x4r __attribute__((ext_vector_type(4)));

// Buffer resource over `bytes` bytes from `base`.
__device__ __forceinline__ u32x4r buf_rsrc(const void* base, uint32_t bytes) {
  const uint64_t a = (uint64_t)base;
  return u32x4r{(uint32_t)a, (uint32_t)(a >> 32) & 0xffffu, bytes, 0x00020000u};
}
#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"  // m0 is set here and used by nothing else
// 16 bytes per lane from the resource at voff + soff into LDS at lds + 16 lane (lds
// wave-uniform).  The range check sees voff only: lanes with voff at or past the resource's size
// write zeros; the uniform soff moves the address.  The compiler does not see these LDS writes:
// they are waited for with explicit vmcnt waits before the barrier that publishes them.
__device__ __forceinline__ void dma16(const u32x4r& rsrc, const bf16_t* lds, uint32_t voff, uint32_t soff) {
  const uint32_t m0 = (uint32_t)(uintptr_t)(const M2_LDS_AS void*)lds;
  asm volatile("s_mov_b32 m0, %0\n\tbuffer_load_dwordx4 %1, %2, %3 offen lds"
               :
               : "s"(m0), "v"(voff), "s"(rsrc), "s"(soff)
               : "m0");
}
#pragma clang diagnostic pop

// Slot of unit 0 of tile row r (r % 16) in 128-byte rows: the 16 rows of a fragment read of
// one unit touch distinct bank groups in every 8-lane and every 16-lane pass.
__device__ __forceinline__ int lswz(int r) { return (r & 6) | ((r ^ (r >> 3)) & 1); }

// s_waitcnt with vmcnt <= n (n < 64) and no wait on the other counters
template <int n>
__device__ __forceinline__ void wait_vm() {
  static_assert(n >= 0 && n < 64, "vmcnt");
  __builtin_amdgcn_s_waitcnt((n & 15) | ((n >> 4) << 14) | (7 << 4) | (15 << 8));
}

__global__ __launch_bounds__(512, 1) void linear_bf16_256_kernel(bf16_t* __restrict__ dst, const bf16_t* __restrict__ x,
                                                                 const bf16_t* __restrict__ w, int M, int N, int K,
                                                                 int tiles_n, int remap) {
  // the operand stages, then (after the K loop) the 256 x 256 bf16 output tile
  __shared__ __attribute__((aligned(1024))) bf16_t smem[2 * LNS * LBM * LBK];
  auto SA = [&](int buf) { return smem + buf * (LBM * LBK); };
  auto SB = [&](int buf) { return smem + (LNS + buf) * (LBM * LBK); };
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane((int)threadIdx.x >> 6);
  const int wm = wave >> 2, wn = wave & 3;

  int t = blockIdx.x;
  if (remap) {
    const int per = gridDim.x / kXcds;
    t = (blockIdx.x % kXcds) * per + blockIdx.x / kXcds;
  }
  const int m0 = (t / tiles_n) * LBM;
  const int n0 = (t % tiles_n) * LBN;
  const int nk = K / LBK;

  // copy instruction a (0..3) of this wave fills tile rows 8 (wave + 8 a) .. +7; lane i: row
  // + i / 8, slot i % 8.  The per-lane offsets are fixed; a step moves the uniform offset, and
  // steps past the end use an empty resource (zeros, no memory access).
  const uint32_t bytes_x = (uint32_t)M * (uint32_t)K * 2u, bytes_w = (uint32_t)N * (uint32_t)K * 2u;
  const u32x4r rsx = buf_rsrc(x, bytes_x), rsw = buf_rsrc(w, bytes_w), rs0 = buf_rsrc(x, 0u);
  uint32_t vx[4], vw[4];
#pragma unroll
  for (int a = 0; a < 4; ++a) {
    const int rr = 8 * (wave + 8 * a) + (lane >> 3);
    const int u = (lane & 7) ^ lswz(rr & 15);
    vx[a] = m0 + rr < M ? 2u * (uint32_t)(m0 + rr) * (uint32_t)K + 16u * (uint32_t)u : bytes_x;
    vw[a] = n0 + rr < N ? 2u * (uint32_t)(n0 + rr) * (uint32_t)K + 16u * (uint32_t)u : bytes_w;
  }
  auto issue = [&](int kt) {
    const int buf = kt & (LNS - 1);
    const bool in = kt < nk;
    const uint32_t so = in ? 128u * (uint32_t)kt : 0u;
#pragma unroll
    for (int a = 0; a < 4; ++a) {
      dma16(in ? rsx : rs0, &SA(buf)[(8 * (wave + 8 * a)) * LBK], vx[a], so);
      dma16(in ? rsw : rs0, &SB(buf)[(8 * (wave + 8 * a)) * LBK], vw[a], so);
    }
  };

  f32x4 acc[8][4];
#pragma unroll
  for (int i = 0; i < 8; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

  // fragment reads: lane l reads row l % 16 of a 16-row tile, unit 4 kk + l / 16
  const int sw = lswz(lane & 15), kq = lane >> 4;
  const int fa = (wm * 128 + (lane & 15)) * LBK, fb = (wn * 64 + (lane & 15)) * LBK;
  auto rd = [&](u32x4 (&af)[8], u32x4 (&bf)[4], int kt, int kk) {
    const int buf = kt & (LNS - 1);
    const int so = 8 * ((4 * kk + kq) ^ sw);
#pragma unroll
    for (int i = 0; i < 8; ++i) af[i] = *reinterpret_cast<const u32x4*>(&SA(buf)[fa + 16 * i * LBK + so]);
#pragma unroll
    for (int j = 0; j < 4; ++j) bf[j] = *reinterpret_cast<const u32x4*>(&SB(buf)[fb + 16 * j * LBK + so]);
  };

  issue(0);
  for (int kt = 0; kt < nk; ++kt) {
    wait_vm<0>();
    __syncthreads();  // stage kt visible; stage kt - 1's buffer no longer read
    issue(kt + 1);
    u32x4 af[2][8], bf[2][4];
    rd(af[0], bf[0], kt, 0);
    rd(af[1], bf[1], kt, 1);
#pragma unroll
    for (int kk = 0; kk < 2; ++kk) {
#pragma unroll
      for (int i = 0; i < 8; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = mfma(bf[kk][j], af[kk][i], acc[i][j]);
    }
    // instruction order: the first half's 12 fragment reads, then the second half's reads one
    // after every two products, then the remaining products.  Left to itself the compiler reads
    // each fragment just before its first product and waits for it there (LDS latency on every
    // fourth product); this order measured 3.5-5 % faster on the layer's shapes.
    __builtin_amdgcn_sched_group_barrier(0x100, 12, 0);  // LDS reads
#pragma unroll
    for (int g = 0; g < 12; ++g) {
      __builtin_amdgcn_sched_group_barrier(0x008, 2, 0);  // MFMA
      __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
    }
    __builtin_amdgcn_sched_group_barrier(0x008, 40, 0);
  }
  wait_vm<0>();  // the zero fill issued in the last step has landed

  // lane l holds dst[row l % 16 of tile i][columns 4 (l / 16) .. +3 of tile j]; the tile row r
  // keeps its 16-byte unit u at unit u ^ (r % 16) of its 512 bytes
  __syncthreads();  // every wave is done reading the operand stages
  char* const tile = reinterpret_cast<char*>(smem);
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const int r = wm * 128 + 16 * i + (lane & 15);
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int c = wn * 64 + 16 * j + 4 * (lane >> 4);
      const f32x4 o = acc[i][j];
      *reinterpret_cast<uint2*>(tile + r * 512 + 16 * ((c >> 3) ^ (r & 15)) + 2 * (c & 7)) =
          make_uint2(pack_bf16x2(o[0], o[1]), pack_bf16x2(o[2], o[3]));
    }
  }
  __syncthreads();
#pragma unroll 4
  for (int q = 0; q < 16; ++q) {
    const int r = wave * 32 + 2 * q + (lane >> 5), u = lane & 31;
    const int m = m0 + r, n = n0 + 8 * u;
    const u32x4 v = *reinterpret_cast<const u32x4*>(tile + r * 512 + 16 * (u ^ (r & 15)));
    if (m < M && n < N) *reinterpret_cast<u32x4*>(dst + (size_t)m * N + n) = v;
  }
}

}  // namespace

// Shapes the projection covers: bf16, K and N multiples of 8 (16-byte loads, 8-byte
// stores), positive sizes, row offsets within 32 bits.
bool linear_supported(int64_t M, int64_t N, int64_t K, int32_t act) {
  return act == MAMBA2_DTYPE_BF16 && M >= 1 && N >= 8 && K >= 8 && N % 8 == 0 && K % 8 == 0 &&
         M * K < ((int64_t)1 << 31) && M * N < ((int64_t)1 << 31) && N * K < ((int64_t)1 << 31);
}

hipError_t launch_linear(void* dst, const void* x, const void* w, int64_t M, int64_t N, int64_t K, hipStream_t st) {
  if (M >= LBM && N >= LBN && K % LBK == 0) {
    const int tm = (int)((M + LBM - 1) / LBM), tn = (int)((N + LBN - 1) / LBN);
    const int64_t nwg = (int64_t)tm * tn;
    const int remap = nwg % kXcds == 0 ? 1 : 0;
    M2_LAUNCH("linear", linear_bf16_256_kernel, dim3((unsigned)nwg), dim3(512), 0, st, (bf16_t*)dst,
              (const bf16_t*)x, (const bf16_t*)w, (int)M, (int)N, (int)K, tn, remap);
    return hipSuccess;
  }
  const int tm = (int)((M + BM - 1) / BM), tn = (int)((N + BN - 1) / BN);
  const int64_t nwg = (int64_t)tm * tn;
  const int remap = nwg % kXcds == 0 ? 1 : 0;
  M2_LAUNCH("linear", linear_bf16_kernel, dim3((unsigned)nwg), dim3(256), 0, st, (bf16_t*)dst, (const bf16_t*)x,
            (const bf16_t*)w, (int)M, (int)N, (int)K, tn, remap);
  return hipSuccess;
}

}  // namespace m2
