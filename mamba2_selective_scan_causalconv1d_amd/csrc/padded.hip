// Padded-batch front end for gfx950: the layer entry of "Granite Mamba2 Inference
// Optimization" takes hidden states [B][Lmax] with an attention mask and must match across
// variable-length padded batches.  The mixer path works on packed runs (a RecurrentBatch),
// so a padded batch is mapped onto one: each batch row's real rows (one contiguous run, at
// the end of every row with left padding or at the start with right padding) are a
// sequence, and the padding rows are not part of it.  pack gathers the real rows of a
// [B][Lmax][row] tensor into [T][row]; unpack scatters [T][row] back to [B][Lmax][row] and
// writes zeros on the padding.
//
// Both are byte copies: one thread per unit (16, 8, 4, 2 or 1 bytes, the largest that divides
// the row and the pointers) of one row; grid (units of a row, padded position, batch row),
// each dimension looping past the grid.  The packed row of padded position j of batch row b
// is cu[b] + j - start(b), start(b) = Lmax - L(b) with left padding, else 0.
#include "common.h"

namespace m2 {
namespace {

constexpr int kThreads = 256;

template <typename U>
__global__ __launch_bounds__(kThreads) void pack_kernel(U* __restrict__ dst, const U* __restrict__ src,
                                                       const int32_t* __restrict__ cu, int B, int Lmax,
                                                       int left, int units) {
  for (int b = blockIdx.z; b < B; b += gridDim.z) {
    const int row0 = cu[b];
    const int L = cu[b + 1] - row0;
    const int j0 = left ? Lmax - L : 0;
    for (int i = blockIdx.y; i < L; i += gridDim.y) {
      const U* s = src + ((size_t)b * Lmax + j0 + i) * units;
      U* d = dst + (size_t)(row0 + i) * units;
      for (int u = blockIdx.x * kThreads + threadIdx.x; u < units; u += gridDim.x * kThreads) d[u] = s[u];
    }
  }
}

template <typename U>
__global__ __launch_bounds__(kThreads) void unpack_kernel(U* __restrict__ dst, const U* __restrict__ src,
                                                         const int32_t* __restrict__ cu, int B, int Lmax,
                                                         int left, int units) {
  for (int b = blockIdx.z; b < B; b += gridDim.z) {
    const int row0 = cu[b];
    const int L = cu[b + 1] - row0;
    const int j0 = left ? Lmax - L : 0;
    for (int j = blockIdx.y; j < Lmax; j += gridDim.y) {
      U* d = dst + ((size_t)b * Lmax + j) * units;
      if (j >= j0 && j < j0 + L) {  // uniform over the workgroup; padding rows read nothing
        const U* s = src + (size_t)(row0 + (j - j0)) * units;
        for (int u = blockIdx.x * kThreads + threadIdx.x; u < units; u += gridDim.x * kThreads) d[u] = s[u];
      } else {
        for (int u = blockIdx.x * kThreads + threadIdx.x; u < units; u += gridDim.x * kThreads) d[u] = U{};
      }
    }
  }
}

unsigned clamp_grid(int64_t n, int64_t cap) { return (unsigned)(n < 1 ? 1 : (n > cap ? cap : n)); }

template <typename U>
hipError_t launch_u(bool pack, void* dst, const void* src, const BatchDev& bd, int32_t Lmax, int32_t left,
                    int64_t row_bytes, hipStream_t st) {
  const int units = (int)(row_bytes / (int64_t)sizeof(U));
  const dim3 grid(clamp_grid((units + kThreads - 1) / kThreads, 64), clamp_grid(Lmax, 65535),
                  clamp_grid(bd.num_seqs, 65535));
  if (pack) {
    M2_LAUNCH("pack_rows", pack_kernel<U>, grid, dim3(kThreads), 0, st, (U*)dst, (const U*)src, bd.cu_seqlens,
              bd.num_seqs, Lmax, left, units);
  } else {
    M2_LAUNCH("unpack_rows", unpack_kernel<U>, grid, dim3(kThreads), 0, st, (U*)dst, (const U*)src,
              bd.cu_seqlens, bd.num_seqs, Lmax, left, units);
  }
  return hipSuccess;
}

}  // namespace

// The largest unit (16, 8, 4, 2 or 1 bytes) that divides the row and both pointers.
int padded_unit_bytes(const void* a, const void* b, int64_t row_bytes) {
  for (int u = 16; u > 1; u >>= 1)
    if (row_bytes % u == 0 && ((uintptr_t)a % u) == 0 && ((uintptr_t)b % u) == 0) return u;
  return 1;
}

hipError_t launch_padded(bool pack, void* dst, const void* src, const BatchDev& bd, int32_t Lmax, int32_t left,
                         int64_t row_bytes, hipStream_t st) {
  switch (padded_unit_bytes(dst, src, row_bytes)) {
    case 16: return launch_u<uint4>(pack, dst, src, bd, Lmax, left, row_bytes, st);
    case 8: return launch_u<uint2>(pack, dst, src, bd, Lmax, left, row_bytes, st);
    case 4: return launch_u<uint32_t>(pack, dst, src, bd, Lmax, left, row_bytes, st);
    case 2: return launch_u<uint16_t>(pack, dst, src, bd, Lmax, left, row_bytes, st);
    default: return launch_u<uint8_t>(pack, dst, src, bd, Lmax, left, row_bytes, st);
  }
}

}  // namespace m2
