// The projections around the mixer path for gfx950: dst[M, N] = x[M, K] . w[N, K]^T in
// bf16 with fp32 accumulation (the layout of a linear layer's weight, one row per output
// feature), one rounding to bf16.  in_proj produces the z, xBC and dt columns (three calls
// on row slices of one weight), out_proj maps the norm's output back to the model width.
//
// MFMA tiling: a 256-thread workgroup computes a 128 x 128 block of dst, each wavefront a
// 64 x 64 quarter as 4 x 4 tiles of v_mfma_f32_16x16x32_bf16.  K advances 64 at a time:
// the x and w rows of the step (16 KiB each) are loaded into registers one step ahead,
// written to a double-buffered LDS tile (rows padded to 144 bytes, so the 16 rows a
// fragment read touches fall in distinct bank groups) and read back as MFMA fragments
// (lane l: row l % 16, k 8 (l / 16) .. +7), one barrier per step.  The product is formed
// as (w x^T)^T: a lane then holds 4 consecutive output columns of one row, stored as 8
// bytes.  Rows and k past the matrix edges are loaded from a clamped address and zeroed.
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

  // global -> register staging: unit i = tid + 256 j is row i / 8, k 8 (i % 8) of the step
  u32x4 ra[4], rb[4];
  auto gload = [&](int k0) {
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int i = tid + 256 * j;
      const int row = i >> 3;
      const int k = k0 + 8 * (i & 7);
      const bool kin = k < K;
      const int kc = kin ? k : K - 8;
      const int ma = min(m0 + row, M - 1), nb = min(n0 + row, N - 1);
      const u32x4 va = *reinterpret_cast<const u32x4*>(x + (size_t)ma * K + kc);
      const u32x4 vb = *reinterpret_cast<const u32x4*>(w + (size_t)nb * K + kc);
      const u32x4 z = {0u, 0u, 0u, 0u};
      ra[j] = (kin && m0 + row < M) ? va : z;
      rb[j] = (kin && n0 + row < N) ? vb : z;
    }
  };
  auto lstore = [&](int buf) {
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int i = tid + 256 * j;
      const int off = (i >> 3) * LDR + 8 * (i & 7);
      *reinterpret_cast<u32x4*>(&sA[buf][off]) = ra[j];
      *reinterpret_cast<u32x4*>(&sB[buf][off]) = rb[j];
    }
  };

  f32x4 acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

  const int nk = (K + BK - 1) / BK;
  gload(0);
  lstore(0);
  __syncthreads();
  const int frow = lane & 15, fk = 8 * (lane >> 4);
  for (int kt = 0; kt < nk; ++kt) {
    const int buf = kt & 1;
    if (kt + 1 < nk) gload((kt + 1) * BK);
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
    if (kt + 1 < nk) lstore(buf ^ 1);
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

}  // namespace

// Shapes the projection covers: bf16, K and N multiples of 8 (16-byte loads, 8-byte
// stores), positive sizes, row offsets within 32 bits.
bool linear_supported(int64_t M, int64_t N, int64_t K, int32_t act) {
  return act == MAMBA2_DTYPE_BF16 && M >= 1 && N >= 8 && K >= 8 && N % 8 == 0 && K % 8 == 0 &&
         M * K < ((int64_t)1 << 31) && M * N < ((int64_t)1 << 31) && N * K < ((int64_t)1 << 31);
}

hipError_t launch_linear(void* dst, const void* x, const void* w, int64_t M, int64_t N, int64_t K, hipStream_t st) {
  const int tm = (int)((M + BM - 1) / BM), tn = (int)((N + BN - 1) / BN);
  const int64_t nwg = (int64_t)tm * tn;
  const int remap = nwg % kXcds == 0 ? 1 : 0;
  M2_LAUNCH("linear", linear_bf16_kernel, dim3((unsigned)nwg), dim3(256), 0, st, (bf16_t*)dst, (const bf16_t*)x,
            (const bf16_t*)w, (int)M, (int)N, (int)K, tn, remap);
  return hipSuccess;
}

}  // namespace m2
