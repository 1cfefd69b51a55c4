// State snapshots and rollback for gfx950: prefix-state snapshots of a prefill run and the
// commit of a verified prefix of a speculative run.
//
// "feat(mamba2): integrate model loading and recurrent inference", section "Notes for
// Reviewers", names prefix-state snapshots and speculative rollback as variants that
// adaptation leaves out.  Their content follows from the recurrence ("feat(backend): Mamba2
// ops, with CPU reference implementations", section "Ops"): a snapshot at boundary b of a
// sequence is the state a run of its first b rows alone would leave in the slots (SSM: h
// after row b; conv: the last K-1 entries of history ++ rows[0, b)).  With a stride E the
// boundaries are E, 2E, ... strictly inside the run; snapshots are packed sequence after
// sequence, sequence s owning floor((L_s - 1) / E) of them from index
// first(s) = sum over earlier sequences of floor((L - 1) / E).
//
// Kernels: the conv snapshots (a gather from the rows and, for boundaries inside the first
// K-1 rows, the slot, so it runs before the conv rewrites the slot); the SSM snapshots of
// a chunked prefill (segments are cut so that every boundary starts a segment, whose
// entering state the inter-segment pass already holds); the commit (slots <- snapshots at
// each sequence's accepted boundary).  Every workgroup computes first(s) itself from the
// device run offsets, so nothing is copied from the host.
#include <algorithm>

#include "common.h"

namespace m2 {
namespace {

constexpr int kThreads = 256;

// first(s): snapshots held by the sequences before s, summed by each wave on its own (no
// barrier: every wave of the workgroup gets the same total).
__device__ int snap_first(const int32_t* __restrict__ cu, int s, int E) {
  int v = 0;
  for (int i = threadIdx.x & 63; i < s; i += 64) v += (cu[i + 1] - cu[i] - 1) / E;
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v += __shfl_xor(v, o, 64);
  return v;
}

typedef uint32_t u32x4v __attribute__((ext_vector_type(4)));

// dst[0, n) = src[0, n) in 16-byte units over the grid's x dimension, four units per thread and
// step (four loads in flight).  Stores stream (the copies are not read back soon); loads stream
// too unless kKeepSrc (a source that later kernels read again).
template <bool kKeepSrc>
__device__ __forceinline__ void copy16(void* dst_, const void* src_, int n) {
  u32x4v* __restrict__ dst = static_cast<u32x4v*>(dst_);
  const u32x4v* __restrict__ src = static_cast<const u32x4v*>(src_);
  constexpr int kPer = 4;
  const int stride = gridDim.x * kThreads * kPer;
  for (int u0 = blockIdx.x * kThreads * kPer + threadIdx.x; u0 < n; u0 += stride) {
    u32x4v v[kPer];
#pragma unroll
    for (int k = 0; k < kPer; ++k)
      if (u0 + k * kThreads < n) v[k] = kKeepSrc ? src[u0 + k * kThreads] : __builtin_nontemporal_load(src + u0 + k * kThreads);
#pragma unroll
    for (int k = 0; k < kPer; ++k)
      if (u0 + k * kThreads < n) __builtin_nontemporal_store(v[k], dst + u0 + k * kThreads);
  }
}

// grid (x: 16-byte units of a snapshot, y: boundary index j - 1, z: sequence), each
// dimension looping when the batch is larger than the grid.
template <typename T>
__global__ __launch_bounds__(kThreads) void conv_snap_kernel(
    T* __restrict__ snaps, const T* __restrict__ x, const T* __restrict__ conv_state,
    const int32_t* __restrict__ cu, const int32_t* __restrict__ slots, const uint8_t* __restrict__ fresh,
    int S, int Dc, int K1, int E) {
  constexpr int V = 16 / sizeof(T);
  const int nv = Dc / V;
  const int units = K1 * nv;
  for (int s = blockIdx.z; s < S; s += gridDim.z) {
    const int first = snap_first(cu, s, E);
    const int L = cu[s + 1] - cu[s];
    const bool is_fresh = fresh[s] != 0;
    const T* hist = conv_state + (size_t)slots[s] * K1 * Dc;
    for (int j = blockIdx.y + 1; (int64_t)j * E < L; j += gridDim.y) {
      const int b = j * E;
      T* out = snaps + (size_t)(first + j - 1) * K1 * Dc;
      for (int u = blockIdx.x * kThreads + threadIdx.x; u < units; u += gridDim.x * kThreads) {
        const int r = u / nv;
        const size_t col = (size_t)(u - r * nv) * V;
        const int idx = b + r;  // entry of history ++ rows
        uint4 v = make_uint4(0, 0, 0, 0);
        if (idx >= K1)
          v = *reinterpret_cast<const uint4*>(x + (size_t)(cu[s] + idx - K1) * Dc + col);
        else if (!is_fresh)
          v = *reinterpret_cast<const uint4*>(hist + (size_t)idx * Dc + col);
        *reinterpret_cast<uint4*>(out + (size_t)r * Dc + col) = v;
      }
    }
  }
}

// grid (x: chunks of all heads' states, y: boundary index j - 1, z: sequence).  The
// boundary jE starts segment jE / seg_len of the sequence; its entering state is the
// snapshot.
__global__ __launch_bounds__(kThreads) void ssm_snap_kernel(float4* __restrict__ snaps,
                                                            const float4* __restrict__ seg_state,
                                                            const int2* __restrict__ seq_info,
                                                            const int32_t* __restrict__ cu, int S, int units,
                                                            int E, int seg_len) {
  for (int s = blockIdx.z; s < S; s += gridDim.z) {
    const int first = snap_first(cu, s, E);
    const int L = cu[s + 1] - cu[s];
    const int seg0 = seq_info[s].x;
    for (int j = blockIdx.y + 1; (int64_t)j * E < L; j += gridDim.y) {
      copy16<true>(snaps + (size_t)(first + j - 1) * units, seg_state + (size_t)(seg0 + (int64_t)j * E / seg_len) * units,
             units);
    }
  }
}

// grid (x: chunks of one sequence's SSM state and of its conv state, z: sequence).
template <typename T>
__global__ __launch_bounds__(kThreads) void commit_kernel(
    uint4* __restrict__ ssm_pool, T* __restrict__ conv_pool, const uint4* __restrict__ ssm_snaps,
    const T* __restrict__ conv_snaps, const int32_t* __restrict__ accepted, const int32_t* __restrict__ cu,
    const int32_t* __restrict__ slots, int S, int ssm_units, int Dc, int K1, int E) {
  constexpr int V = 16 / sizeof(T);
  const int conv_units = K1 * Dc / V;
  for (int s = blockIdx.z; s < S; s += gridDim.z) {
    const int first = snap_first(cu, s, E);
    const int L = cu[s + 1] - cu[s];
    const int m = accepted[s];
    if (m < 1 || m >= L || m % E != 0) continue;  // uniform over the workgroup
    const size_t idx = (size_t)first + m / E - 1;
    const size_t slot = (size_t)slots[s];
    if (ssm_snaps) copy16<false>(ssm_pool + slot * ssm_units, ssm_snaps + idx * ssm_units, ssm_units);
    if (conv_snaps)
      copy16<false>(conv_pool + slot * K1 * Dc, conv_snaps + idx * K1 * Dc, conv_units);
  }
}

unsigned clamp_grid(int64_t n, int64_t cap) { return (unsigned)(n < 1 ? 1 : (n > cap ? cap : n)); }

}  // namespace

int64_t snapshot_count(const mamba2_recurrent_batch* rb, int32_t E) {
  int64_t n = 0;
  for (int s = 0; s < rb->num_seqs; ++s) n += (rb->run_lengths[s] - 1) / E;
  return n;
}

int32_t snapshot_max_per_seq(const mamba2_recurrent_batch* rb, int32_t E) {
  int32_t m = 0;
  for (int s = 0; s < rb->num_seqs; ++s) m = std::max(m, (rb->run_lengths[s] - 1) / E);
  return m;
}

hipError_t launch_conv_snapshots(void* snaps, const void* x, const void* conv_state, const BatchDev& bd,
                                 int32_t maxj, int32_t Dc, int32_t K, int32_t E, int32_t act, hipStream_t st) {
  if (maxj == 0 || bd.num_seqs == 0) return hipSuccess;
  const int V = act == MAMBA2_DTYPE_BF16 ? 8 : 4;
  const int64_t units = (int64_t)(K - 1) * Dc / V;
  const dim3 grid(clamp_grid((units + kThreads - 1) / kThreads, 64), clamp_grid(maxj, 65535),
                  clamp_grid(bd.num_seqs, 65535));
  if (act == MAMBA2_DTYPE_BF16) {
    M2_LAUNCH("conv_snapshots", conv_snap_kernel<bf16_t>, grid, dim3(kThreads), 0, st, (bf16_t*)snaps,
              (const bf16_t*)x, (const bf16_t*)conv_state, bd.cu_seqlens, bd.slots, bd.fresh, bd.num_seqs, Dc,
              K - 1, E);
  } else {
    M2_LAUNCH("conv_snapshots", conv_snap_kernel<float>, grid, dim3(kThreads), 0, st, (float*)snaps,
              (const float*)x, (const float*)conv_state, bd.cu_seqlens, bd.slots, bd.fresh, bd.num_seqs, Dc,
              K - 1, E);
  }
  return hipSuccess;
}

hipError_t launch_ssm_snapshots(const ScanArgs& a, float* snaps, int32_t maxj, int32_t E, hipStream_t st) {
  if (maxj == 0 || a.bd.num_seqs == 0) return hipSuccess;
  const int64_t units = (int64_t)a.dims.nheads * a.dims.headdim * a.dims.d_state / 4;
  const dim3 grid(clamp_grid((units + 4 * kThreads - 1) / (4 * kThreads), 1024), clamp_grid(maxj, 65535),
                  clamp_grid(a.bd.num_seqs, 65535));
  M2_LAUNCH("ssm_snapshots", ssm_snap_kernel, grid, dim3(kThreads), 0, st, (float4*)snaps,
            (const float4*)(a.ws + a.lay.off_seg_state), (const int2*)(a.ws + a.lay.off_seq_info),
            a.bd.cu_seqlens, a.bd.num_seqs, (int)units, E, a.lay.seg_len);
  return hipSuccess;
}

hipError_t launch_commit(float* ssm_state, void* conv_state, const float* ssm_snaps, const void* conv_snaps,
                         const int32_t* accepted, const BatchDev& bd, const mamba2_dims& dm, int32_t E,
                         hipStream_t st) {
  if (bd.num_seqs == 0) return hipSuccess;
  const int Dc = dm.nheads * dm.headdim + 2 * dm.ngroups * dm.d_state;
  const int K1 = dm.conv_kernel - 1;
  const int V = dm.act_dtype == MAMBA2_DTYPE_BF16 ? 8 : 4;
  const int64_t ssm_units = (int64_t)dm.nheads * dm.headdim * dm.d_state / 4;
  const int64_t units = (ssm_snaps ? ssm_units : 0) + (conv_snaps ? (int64_t)K1 * Dc / V : 0);
  const dim3 grid(clamp_grid((units + 4 * kThreads - 1) / (4 * kThreads), 1024), 1, clamp_grid(bd.num_seqs, 65535));
  if (dm.act_dtype == MAMBA2_DTYPE_BF16) {
    M2_LAUNCH("commit_snapshots", commit_kernel<bf16_t>, grid, dim3(kThreads), 0, st, (uint4*)ssm_state,
              (bf16_t*)conv_state, (const uint4*)ssm_snaps, (const bf16_t*)conv_snaps, accepted, bd.cu_seqlens,
              bd.slots, bd.num_seqs, (int)ssm_units, Dc, K1, E);
  } else {
    M2_LAUNCH("commit_snapshots", commit_kernel<float>, grid, dim3(kThreads), 0, st, (uint4*)ssm_state,
              (float*)conv_state, (const uint4*)ssm_snaps, (const float*)conv_snaps, accepted, bd.cu_seqlens,
              bd.slots, bd.num_seqs, (int)ssm_units, Dc, K1, E);
  }
  return hipSuccess;
}

}  // namespace m2
