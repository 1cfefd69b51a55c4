// The projections around the mixer path for gfx950: dst[M, N] = x[M, K] . w[N, K]^T in
// bf16 with fp32 accumulation (the layout of a linear layer's weight, one row per output
// feature), one rounding to bf16.  in_proj produces the z, xBC and dt columns (three calls
// on row slices of one weight), out_proj maps the norm's output back to the model width.
//
// MFMA tiling: a 256-thread workgroup computes a 128 x 128 block of dst, each wavefront a
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
// For M, N >= 256: a 512-thread workgroup computes a 256 x 256 block of dst, wavefront (wm, wn)
// a 128 x 64 part of it (8 x 4 MFMA tiles, 128 accumulators per lane).  K advances 32 at a
// time through four LDS stages of 32 KiB (the step's 256 x rows and 256 w rows, 64 bytes each):
// the copies of step k + 3 are issued as step k is contracted, one barrier per step.  The
// copies are buffer loads that write LDS directly (no registers, no LDS stores): each
// instruction fills 1 KiB (16 rows x 4 units of 16 bytes) and each lane fetches the global unit
// that lands in its slot.  Units are stored XOR-swizzled: unit u of tile row r sits in slot
// u ^ ((r / 4) % 4), so the 16 rows a fragment read touches fall in distinct bank groups.
// Rows past M or N and k past K read as zero (out-of-range buffer offsets).

constexpr int LBM = 256, LBN = 256, LBK = 32, LNS = 4;

#define M2_LDS_AS __attribute__((address_space(3)))
typedef uint32_t u32x4r __attribute__((ext_vector_type(4)));
#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"  // m0 is set here and used by nothing else
// 16 bytes per lane from base + voff into LDS at lds + 16 lane (lds wave-uniform); offsets at or
// past `bytes` write zeros.  The compiler does not see these LDS writes: they are waited for with
// explicit vmcnt waits before the barrier that publishes them.
__device__ __forceinline__ void dma16(const void* base, uint32_t bytes, const bf16_t* lds, uint32_t voff) {
  const uint64_t a = (uint64_t)base;
  const u32x4r rsrc = {(uint32_t)a, (uint32_t)(a >> 32) & 0xffffu, bytes, 0x00020000u};
  const uint32_t m0 = (uint32_t)(uintptr_t)(const M2_LDS_AS void*)lds;
  asm volatile("s_mov_b32 m0, %0\n\tbuffer_load_dwordx4 %1, %2, 0 offen lds"
               :
               : "s"(m0), "v"(voff), "s"(rsrc)
               : "m0");
}
#pragma clang diagnostic pop

// s_waitcnt with vmcnt <= n (n < 64) and no wait on the other counters
template <int n>
__device__ __forceinline__ void wait_vm() {
  static_assert(n >= 0 && n < 64, "vmcnt");
  __builtin_amdgcn_s_waitcnt((n & 15) | ((n >> 4) << 14) | (7 << 4) | (15 << 8));
}

__global__ __launch_bounds__(512, 1) void linear_bf16_256_kernel(bf16_t* __restrict__ dst, const bf16_t* __restrict__ x,
                                                                 const bf16_t* __restrict__ w, int M, int N, int K,
                                                                 int tiles_n, int remap) {
  __shared__ __attribute__((aligned(1024))) bf16_t sA[LNS][LBM * LBK];
  __shared__ __attribute__((aligned(1024))) bf16_t sB[LNS][LBN * LBK];
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
  const int nk = (K + LBK - 1) / LBK;

  // copy instructions of this wave: tile rows 16 j .. 16 j + 15, j = wave and wave + 8, of x and w
  const uint32_t bytes_x = (uint32_t)M * (uint32_t)K * 2u, bytes_w = (uint32_t)N * (uint32_t)K * 2u;
  const int crow = lane >> 2;                      // row within the instruction's 16
  const int cunit = (lane & 3) ^ (lane >> 4);      // global unit fetched into slot lane % 4
  const int rx0 = m0 + 16 * wave + crow, rx1 = rx0 + 128;
  const int rw0 = n0 + 16 * wave + crow, rw1 = rw0 + 128;
  auto issue = [&](int kt) {
    const int buf = kt & (LNS - 1);
    const int k = kt * LBK + 8 * cunit;
    const bool kin = kt < nk && k < K;
    const uint32_t ko = 2u * (uint32_t)k;
    const uint32_t ox0 = (kin && rx0 < M) ? 2u * (uint32_t)rx0 * (uint32_t)K + ko : bytes_x;
    const uint32_t ox1 = (kin && rx1 < M) ? 2u * (uint32_t)rx1 * (uint32_t)K + ko : bytes_x;
    const uint32_t ow0 = (kin && rw0 < N) ? 2u * (uint32_t)rw0 * (uint32_t)K + ko : bytes_w;
    const uint32_t ow1 = (kin && rw1 < N) ? 2u * (uint32_t)rw1 * (uint32_t)K + ko : bytes_w;
    dma16(x, bytes_x, &sA[buf][(16 * wave) * LBK], ox0);
    dma16(x, bytes_x, &sA[buf][(16 * wave + 128) * LBK], ox1);
    dma16(w, bytes_w, &sB[buf][(16 * wave) * LBK], ow0);
    dma16(w, bytes_w, &sB[buf][(16 * wave + 128) * LBK], ow1);
  };

  f32x4 acc[8][4];
#pragma unroll
  for (int i = 0; i < 8; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

  // fragment reads: lane l reads row l % 16 of a 16-row tile, unit l / 16, from slot
  // (l / 16) ^ ((l % 16) / 4)
  const int frag = (lane & 15) * LBK + 8 * ((lane >> 4) ^ ((lane & 15) >> 2));
  const int fa = (wm * 128) * LBK + frag, fb = (wn * 64) * LBK + frag;

  issue(0);
  issue(1);
  issue(2);
  for (int kt = 0; kt < nk; ++kt) {
    wait_vm<8>();  // this wave's copies of step kt have landed (steps kt + 1, kt + 2 may be in flight)
    __syncthreads();  // everyone's have; step kt - 1's stage is no longer read
    issue(kt + 3);
    const int buf = kt & (LNS - 1);
    u32x4 af[8], bf[4];
#pragma unroll
    for (int i = 0; i < 8; ++i) af[i] = *reinterpret_cast<const u32x4*>(&sA[buf][fa + 16 * i * LBK]);
#pragma unroll
    for (int j = 0; j < 4; ++j) bf[j] = *reinterpret_cast<const u32x4*>(&sB[buf][fb + 16 * j * LBK]);
#pragma unroll
    for (int i = 0; i < 8; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j) acc[i][j] = mfma(bf[j], af[i], acc[i][j]);
  }
  wait_vm<0>();  // the copies issued past the last step (zero fills) land before the workgroup ends

  // lane l holds dst[row l % 16 of tile i][columns 4 (l / 16) .. +3 of tile j]
  const int frow = lane & 15;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const int m = m0 + wm * 128 + 16 * i + frow;
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

}  // namespace

// Shapes the projection covers: bf16, K and N multiples of 8 (16-byte loads, 8-byte
// stores), positive sizes, row offsets within 32 bits.
bool linear_supported(int64_t M, int64_t N, int64_t K, int32_t act) {
  return act == MAMBA2_DTYPE_BF16 && M >= 1 && N >= 8 && K >= 8 && N % 8 == 0 && K % 8 == 0 &&
         M * K < ((int64_t)1 << 31) && M * N < ((int64_t)1 << 31) && N * K < ((int64_t)1 << 31);
}

hipError_t launch_linear(void* dst, const void* x, const void* w, int64_t M, int64_t N, int64_t K, hipStream_t st) {
  if (M >= LBM && N >= LBN) {
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
