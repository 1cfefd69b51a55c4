// Gated RMSNorm for gfx950: out = g / sqrt(mean_group(g^2) + eps) * w, g = x * silu(z).
//
// Operation: "feat(backend): Mamba2 ops, with CPU reference implementations", section
// "Ops", GatedRMSNorm (the gate before the norm, the RMS per group of d_inner/groups
// columns).
//
// Mapping: one wavefront per (row, group).  Each lane holds up to kMaxVec 16-byte
// vectors of x and z in registers (the group is read once and written once: a
// streaming HBM-bound kernel), the sum of squares is a wave reduction.
#include "common.h"

namespace m2 {
namespace {

constexpr int kMaxVec = 8;

template <typename T>
__global__ __launch_bounds__(256) void gated_rmsnorm_kernel(T* __restrict__ dst,
                                                            const T* __restrict__ x,
                                                            const T* __restrict__ z,
                                                            const float* __restrict__ w,
                                                            int groups, float eps, int rows,
                                                            int Di) {
  constexpr int V = Act<T>::kVec;
  const int lane = threadIdx.x & 63;
  const int64_t unit = (int64_t)blockIdx.x * (blockDim.x >> 6) + (threadIdx.x >> 6);
  if (unit >= (int64_t)rows * groups) return;
  const int row = (int)(unit / groups);
  const int q = (int)(unit % groups);
  const int gs = Di / groups;
  const int nv = gs / V;
  const size_t base = (size_t)row * Di + (size_t)q * gs;

  float g[kMaxVec][V];
  float ss = 0.f;
#pragma unroll
  for (int k = 0; k < kMaxVec; ++k) {
    const int vi = lane + 64 * k;
    if (vi < nv) {
      float xf[V], zf[V];
      Act<T>::unpack(*reinterpret_cast<const uint4*>(x + base + (size_t)vi * V), xf);
      Act<T>::unpack(*reinterpret_cast<const uint4*>(z + base + (size_t)vi * V), zf);
#pragma unroll
      for (int i = 0; i < V; ++i) {
        g[k][i] = xf[i] * silu_f32(zf[i]);
        ss = fmaf(g[k][i], g[k][i], ss);
      }
    }
  }
  ss = wave_sum(ss);
  const float inv = rsqrtf(ss / (float)gs + eps);
#pragma unroll
  for (int k = 0; k < kMaxVec; ++k) {
    const int vi = lane + 64 * k;
    if (vi < nv) {
      const float* wp = w + (size_t)q * gs + (size_t)vi * V;
      float out[V];
#pragma unroll
      for (int i = 0; i < V; ++i) out[i] = g[k][i] * inv * wp[i];
      *reinterpret_cast<uint4*>(dst + base + (size_t)vi * V) = Act<T>::pack(out);
    }
  }
}

// Groups wider than 64 * kMaxVec vectors: two passes over the group (the second
// pass re-reads x and z, normally from L2).
template <typename T>
__global__ __launch_bounds__(256) void gated_rmsnorm_wide_kernel(T* __restrict__ dst,
                                                                 const T* __restrict__ x,
                                                                 const T* __restrict__ z,
                                                                 const float* __restrict__ w,
                                                                 int groups, float eps, int rows,
                                                                 int Di) {
  constexpr int V = Act<T>::kVec;
  const int lane = threadIdx.x & 63;
  const int64_t unit = (int64_t)blockIdx.x * (blockDim.x >> 6) + (threadIdx.x >> 6);
  if (unit >= (int64_t)rows * groups) return;
  const int row = (int)(unit / groups);
  const int q = (int)(unit % groups);
  const int gs = Di / groups;
  const int nv = gs / V;
  const size_t base = (size_t)row * Di + (size_t)q * gs;
  float ss = 0.f;
  for (int vi = lane; vi < nv; vi += 64) {
    float xf[V], zf[V];
    Act<T>::unpack(*reinterpret_cast<const uint4*>(x + base + (size_t)vi * V), xf);
    Act<T>::unpack(*reinterpret_cast<const uint4*>(z + base + (size_t)vi * V), zf);
#pragma unroll
    for (int i = 0; i < V; ++i) {
      const float gv = xf[i] * silu_f32(zf[i]);
      ss = fmaf(gv, gv, ss);
    }
  }
  ss = wave_sum(ss);
  const float inv = rsqrtf(ss / (float)gs + eps);
  for (int vi = lane; vi < nv; vi += 64) {
    float xf[V], zf[V], out[V];
    Act<T>::unpack(*reinterpret_cast<const uint4*>(x + base + (size_t)vi * V), xf);
    Act<T>::unpack(*reinterpret_cast<const uint4*>(z + base + (size_t)vi * V), zf);
    const float* wp = w + (size_t)q * gs + (size_t)vi * V;
#pragma unroll
    for (int i = 0; i < V; ++i) out[i] = xf[i] * silu_f32(zf[i]) * inv * wp[i];
    *reinterpret_cast<uint4*>(dst + base + (size_t)vi * V) = Act<T>::pack(out);
  }
}

template <typename T>
hipError_t launch_t(void* dst, const void* x, const void* z, const float* w, int32_t groups,
                    float eps, int32_t rows, int32_t Di, hipStream_t st) {
  constexpr int V = Act<T>::kVec;
  const int64_t units = (int64_t)rows * groups;
  const dim3 grid((unsigned)((units + 3) / 4));
  if ((Di / groups) / V <= 64 * kMaxVec) {
    M2_LAUNCH("gated_rmsnorm", gated_rmsnorm_kernel<T>, grid, dim3(256), 0, st, (T*)dst,
              (const T*)x, (const T*)z, w, groups, eps, rows, Di);
  } else {
    M2_LAUNCH("gated_rmsnorm_wide", gated_rmsnorm_wide_kernel<T>, grid, dim3(256), 0, st, (T*)dst,
              (const T*)x, (const T*)z, w, groups, eps, rows, Di);
  }
  return hipSuccess;
}

}  // namespace

hipError_t launch_gated_rmsnorm(void* dst, const void* x, const void* z, const float* w,
                                int32_t groups, float eps, int32_t rows, int32_t Di, int32_t act,
                                hipStream_t st) {
  if (act == MAMBA2_DTYPE_BF16) return launch_t<bf16_t>(dst, x, z, w, groups, eps, rows, Di, st);
  return launch_t<float>(dst, x, z, w, groups, eps, rows, Di, st);
}

}  // namespace m2
