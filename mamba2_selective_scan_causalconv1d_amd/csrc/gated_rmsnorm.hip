// Gated RMSNorm for gfx950: out = g / sqrt(mean_group(g^2) + eps) * w, g = x * silu(z).
//
// Operation: "feat(backend): Mamba2 ops, with CPU reference implementations", section
// "Ops", GatedRMSNorm (the gate before the norm, the RMS per group of d_inner/groups
// columns).
//
// Mapping (row kernel): one wavefront per row, the row held in registers (read once,
// written once: a streaming HBM-bound kernel).  Each group owns a contiguous run of
// L = 64 / groups lanes, and its 16-byte vectors are dealt to those lanes round robin,
// so every load instruction touches whole 128-byte lines and the group's sum of squares
// is a DPP / swizzle reduction over L lanes.  The weights are loaded before the reduction.
// Four rows per workgroup, rows streamed with non-temporal accesses.  A launch of fewer than
// 4096 rows (a decode step) is latency-bound: it takes one workgroup per row whose waves share
// the row's vectors (each lane gates one vector), the waves' group sums added in wave order
// through LDS.  Shapes that do not fit (groups not dividing 64, rows not a multiple of 64
// vectors) use the unit kernel: one wavefront per (row, group).
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

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

// The weight vectors are loaded before the row's reduction, so each wave waits on one round of
// loads instead of two (203 -> 198 us on a 65536 x 3072 launch).  The rows are streamed: x, z
// and dst use non-temporal accesses (each byte is touched once), which keeps the stream from
// displacing cached data.
template <typename T, int NVPL>
__global__ __launch_bounds__(256) void gated_rmsnorm_row_kernel(T* __restrict__ dst, const T* __restrict__ x,
                                                                const T* __restrict__ z,
                                                                const float* __restrict__ w, int lanes_per_group,
                                                                int log2_lpg, float eps, float inv_gs, int rows,
                                                                int Di) {
  constexpr int V = Act<T>::kVec;
  const int lane = threadIdx.x & 63;
  const int row = blockIdx.x * (blockDim.x >> 6) + (threadIdx.x >> 6);
  if (row >= rows) return;
  const int q = lane >> log2_lpg;                 // this lane's group
  const int jl = lane & (lanes_per_group - 1);    // its place in the group's lanes
  const int gv = NVPL * lanes_per_group;          // vectors per group
  const size_t base = (size_t)row * Di;
  float wf[NVPL][V];
  auto load_w = [&](int k) {
    const int vi = q * gv + jl + lanes_per_group * k;
    const float4* wp = reinterpret_cast<const float4*>(w + (size_t)vi * V);
#pragma unroll
    for (int i = 0; i < V / 4; ++i) {
      const float4 t4 = wp[i];
      wf[k][4 * i] = t4.x;
      wf[k][4 * i + 1] = t4.y;
      wf[k][4 * i + 2] = t4.z;
      wf[k][4 * i + 3] = t4.w;
    }
  };
#pragma unroll
  for (int k = 0; k < NVPL; ++k) load_w(k);
  auto load_row = [&](const T* p) -> uint4 {
    const u32x4 v = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
    return make_uint4(v.x, v.y, v.z, v.w);
  };
  float g[NVPL][V];
  float ss = 0.f;
#pragma unroll
  for (int k = 0; k < NVPL; ++k) {
    const int vi = q * gv + jl + lanes_per_group * k;
    float xf[V], zf[V];
    Act<T>::unpack(load_row(x + base + (size_t)vi * V), xf);
    Act<T>::unpack(load_row(z + base + (size_t)vi * V), zf);
#pragma unroll
    for (int i = 0; i < V; ++i) {
      g[k][i] = xf[i] * silu_f32(zf[i]);
      ss = fmaf(g[k][i], g[k][i], ss);
    }
  }
  ss = group_sum(ss, lanes_per_group);
  const float inv = rsqrtf(ss * inv_gs + eps);
#pragma unroll
  for (int k = 0; k < NVPL; ++k) {
    const int vi = q * gv + jl + lanes_per_group * k;
    float out[V];
#pragma unroll
    for (int i = 0; i < V; ++i) out[i] = g[k][i] * inv * wf[k][i];
    const uint4 pv = Act<T>::pack(out);
    __builtin_nontemporal_store(u32x4{pv.x, pv.y, pv.z, pv.w}, reinterpret_cast<u32x4*>(dst + base + (size_t)vi * V));
  }
}

// A row per workgroup of NVPL waves (few rows): lane slot (q, jl) of wave k holds the vector
// that the row kernel's lane holds as its k-th, so the lanes of a group are the same and
// every wave's group sum is a reduction over them; the NVPL sums go through LDS and are added
// in wave order (the same order in every lane of the group).
template <typename T, int NVPL>
__global__ __launch_bounds__(64 * NVPL) void gated_rmsnorm_split_kernel(T* __restrict__ dst, const T* __restrict__ x,
                                                                       const T* __restrict__ z,
                                                                       const float* __restrict__ w,
                                                                       int lanes_per_group, int log2_lpg, float eps,
                                                                       float inv_gs, int Di) {
  constexpr int V = Act<T>::kVec;
  __shared__ float part[NVPL][64];
  const int lane = threadIdx.x & 63;
  const int k = threadIdx.x >> 6;
  const int q = lane >> log2_lpg;
  const int jl = lane & (lanes_per_group - 1);
  const int vi = q * NVPL * lanes_per_group + jl + lanes_per_group * k;
  const size_t at = (size_t)blockIdx.x * Di + (size_t)vi * V;
  float wf[V], xf[V], zf[V];
  const float4* wp = reinterpret_cast<const float4*>(w + (size_t)vi * V);
#pragma unroll
  for (int i = 0; i < V / 4; ++i) {
    const float4 t4 = wp[i];
    wf[4 * i] = t4.x;
    wf[4 * i + 1] = t4.y;
    wf[4 * i + 2] = t4.z;
    wf[4 * i + 3] = t4.w;
  }
  Act<T>::unpack(*reinterpret_cast<const uint4*>(x + at), xf);
  Act<T>::unpack(*reinterpret_cast<const uint4*>(z + at), zf);
  float g[V];
  float ss = 0.f;
#pragma unroll
  for (int i = 0; i < V; ++i) {
    g[i] = xf[i] * silu_f32(zf[i]);
    ss = fmaf(g[i], g[i], ss);
  }
  part[k][lane] = group_sum(ss, lanes_per_group);
  __syncthreads();
  float tot = part[0][lane];
#pragma unroll
  for (int j = 1; j < NVPL; ++j) tot += part[j][lane];
  const float inv = rsqrtf(tot * inv_gs + eps);
  float out[V];
#pragma unroll
  for (int i = 0; i < V; ++i) out[i] = g[i] * inv * wf[i];
  *reinterpret_cast<uint4*>(dst + at) = Act<T>::pack(out);
}

template <typename T, int NVPL>
hipError_t launch_row(void* dst, const void* x, const void* z, const float* w, int32_t groups, float eps,
                      int32_t rows, int32_t Di, hipStream_t st) {
  const int lpg = 64 / groups;
  int log2_lpg = 0;
  while ((1 << log2_lpg) < lpg) ++log2_lpg;
  const float inv_gs = 1.f / (float)(Di / groups);
  if (rows < 4096) {
    // few rows (a decode step): a workgroup of NVPL waves per row
    M2_LAUNCH("gated_rmsnorm", (gated_rmsnorm_split_kernel<T, NVPL>), dim3((unsigned)rows), dim3(64 * NVPL), 0, st,
              (T*)dst, (const T*)x, (const T*)z, w, lpg, log2_lpg, eps, inv_gs, Di);
    return hipSuccess;
  }
  const dim3 grid((unsigned)((rows + 3) / 4));
  M2_LAUNCH("gated_rmsnorm", (gated_rmsnorm_row_kernel<T, NVPL>), grid, dim3(256), 0, st, (T*)dst,
            (const T*)x, (const T*)z, w, lpg, log2_lpg, eps, inv_gs, rows, Di);
  return hipSuccess;
}

template <typename T>
hipError_t launch_t(void* dst, const void* x, const void* z, const float* w, int32_t groups,
                    float eps, int32_t rows, int32_t Di, hipStream_t st) {
  constexpr int V = Act<T>::kVec;
  const int nv_row = Di / V;
  if (64 % groups == 0 && nv_row % 64 == 0) {
    switch (nv_row / 64) {
      case 1: return launch_row<T, 1>(dst, x, z, w, groups, eps, rows, Di, st);
      case 2: return launch_row<T, 2>(dst, x, z, w, groups, eps, rows, Di, st);
      case 3: return launch_row<T, 3>(dst, x, z, w, groups, eps, rows, Di, st);
      case 4: return launch_row<T, 4>(dst, x, z, w, groups, eps, rows, Di, st);
      case 6: return launch_row<T, 6>(dst, x, z, w, groups, eps, rows, Di, st);
      case 8: return launch_row<T, 8>(dst, x, z, w, groups, eps, rows, Di, st);
      default: break;
    }
  }
  const int64_t units = (int64_t)rows * groups;
  const dim3 grid((unsigned)((units + 3) / 4));
  if ((Di / groups) / V <= 64 * kMaxVec) {
    M2_LAUNCH("gated_rmsnorm_unit", gated_rmsnorm_kernel<T>, grid, dim3(256), 0, st, (T*)dst,
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
