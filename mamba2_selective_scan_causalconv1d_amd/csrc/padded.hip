// Padded-batch front end for gfx950: the layer entry of "Granite Mamba2 Inference
// Optimization" takes hidden states [B][Lmax] with an attention mask and must match across
// variable-length padded batches.  The mixer path works on packed runs (a RecurrentBatch),
// so a padded batch is mapped onto one: each batch row's real rows (one contiguous run, at
// the end of every row with left padding or at the start with right padding) are a
// sequence, and the padding rows are not part of it.  pack gathers the real rows of a
// [B][Lmax][row] tensor into [T][row]; unpack scatters [T][row] back to [B][Lmax][row] and
// writes zeros on the padding.
//
// Both are byte copies.  The real rows of a batch row are contiguous in the padded layout as
// well as in the packed one: packed unit e of batch row b (cu[b] units <= e < cu[b + 1] units,
// counting row by row) is padded unit e + delta(b), delta(b) = (b Lmax + start(b) - cu[b]) units,
// start(b) = Lmax - L(b) with left padding, else 0.  pack copies each batch row's run as one
// contiguous span: workgroup (x, b) takes span chunk x of batch row b (grid y over the batch
// rows, strided past the grid's limit), so the row is a uniform index and no lookup precedes
// the loads.  unpack walks the padded units flat over the whole tensor (zero outside [start(b),
// start(b) + L(b))).  Units are 16, 8, 4, 2 or 1 bytes (the largest that divides the row and the
// pointers); unpack moves four per thread and step, pack one (a workgroup per 4 KiB of a run:
// 30 us for the varlen batch's xBC rows, the rate of a plain device copy, against 37 us with four
// units per thread and 66 us with eight).
#include "common.h"

namespace m2 {
namespace {

constexpr int kThreads = 256;
constexpr int kPer = 4;  // units per thread and step (unpack)

// Batch row b's run: units [cu[b] units, cu[b + 1] units) of dst from the same count of units of
// src starting at (b Lmax + start(b)) units.  Workgroup x copies chunks x, x + gridDim.x, ... of
// kThreads units (one per thread) of each of its rows.
template <typename U>
__global__ __launch_bounds__(kThreads) void pack_kernel(U* __restrict__ dst, const U* __restrict__ src,
                                                       const int32_t* __restrict__ cu, int B, int Lmax,
                                                       int left, int64_t units) {
  for (int b = blockIdx.y; b < B; b += gridDim.y) {
    const int c0 = cu[b], L = cu[b + 1] - c0;
    const int64_t n = (int64_t)L * units;
    const U* s = src + ((int64_t)b * Lmax + (left ? Lmax - L : 0)) * units;
    U* d = dst + (int64_t)c0 * units;
    for (int64_t e = (int64_t)blockIdx.x * kThreads + threadIdx.x; e < n; e += (int64_t)gridDim.x * kThreads)
      d[e] = s[e];
  }
}

template <typename U>
__global__ __launch_bounds__(kThreads) void unpack_kernel(U* __restrict__ dst, const U* __restrict__ src,
                                                         const int32_t* __restrict__ cu, int B, int Lmax,
                                                         int left, int64_t units) {
  const int64_t per_row = (int64_t)Lmax * units;
  const int64_t n = (int64_t)B * per_row;
  const int64_t stride = (int64_t)gridDim.x * kThreads * kPer;
  // real units of batch row b: [first, first + L units), read from packed unit e - first + cu[b] units
  auto span = [&](int b, int64_t& first, int64_t& last, int64_t& off) {
    const int L = cu[b + 1] - cu[b];
    first = ((int64_t)b * Lmax + (left ? Lmax - L : 0)) * units;
    last = first + (int64_t)L * units;
    off = (int64_t)cu[b] * units - first;
  };
  for (int64_t c0 = (int64_t)blockIdx.x * kThreads * kPer; c0 < n; c0 += stride) {
    const int b0 = (int)(c0 / per_row);
    const int64_t end0 = (int64_t)(b0 + 1) * per_row;
    int64_t f0, l0, o0;
    span(b0, f0, l0, o0);
    U v[kPer];
#pragma unroll
    for (int k = 0; k < kPer; ++k) {
      const int64_t e = c0 + threadIdx.x + (int64_t)k * kThreads;
      v[k] = U{};
      if (e < n) {
        int64_t f = f0, l = l0, o = o0;
        if (e >= end0) {
          int b = b0 + 1;
          while ((int64_t)(b + 1) * per_row <= e) ++b;
          span(b, f, l, o);
        }
        if (e >= f && e < l) v[k] = src[e + o];
      }
    }
#pragma unroll
    for (int k = 0; k < kPer; ++k) {
      const int64_t e = c0 + threadIdx.x + (int64_t)k * kThreads;
      if (e < n) dst[e] = v[k];
    }
  }
}

unsigned clamp_grid(int64_t n, int64_t cap) { return (unsigned)(n < 1 ? 1 : (n > cap ? cap : n)); }

template <typename U>
hipError_t launch_u(bool pack, void* dst, const void* src, const BatchDev& bd, int32_t Lmax, int32_t left,
                    int64_t row_bytes, hipStream_t st) {
  const int64_t units = row_bytes / (int64_t)sizeof(U);
  if (pack) {
    // chunks of the longest possible run (Lmax rows) over x, batch rows over y
    const dim3 grid(clamp_grid(((int64_t)Lmax * units + kThreads - 1) / kThreads, 65535), clamp_grid(bd.num_seqs, 65535));
    M2_LAUNCH("pack_rows", pack_kernel<U>, grid, dim3(kThreads), 0, st, (U*)dst, (const U*)src, bd.cu_seqlens,
              bd.num_seqs, Lmax, left, units);
    return hipSuccess;
  }
  const int64_t n = (int64_t)bd.num_seqs * Lmax * units;
  const dim3 grid(clamp_grid((n + kThreads * kPer - 1) / (kThreads * kPer), 4096));
  M2_LAUNCH("unpack_rows", unpack_kernel<U>, grid, dim3(kThreads), 0, st, (U*)dst, (const U*)src, bd.cu_seqlens,
            bd.num_seqs, Lmax, left, units);
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
