// Internal declarations of the gfx950 kernels and their host launchers.
// Device helpers for bf16 storage, wave-level reductions and the workspace layout
// of the chunked scan.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "../../include/mamba2.h"

namespace m2 {

// ------------------------------------------------------------------ storage

typedef uint16_t bf16_t;  // raw bf16 bits

__device__ __forceinline__ float bf16_to_f32(uint32_t b) { return __uint_as_float(b << 16); }

// fp32 -> bf16 by the gfx950 conversion instruction (v_cvt_pk_bf16_f32: round to nearest
// even, two values per instruction).
typedef __bf16 bf16x2_hw __attribute__((ext_vector_type(2)));
typedef float f32x2_hw __attribute__((ext_vector_type(2)));

// two fp32 -> packed bf16x2 (lo in bits 0..15)
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  return __builtin_bit_cast(uint32_t, __builtin_convertvector((f32x2_hw){lo, hi}, bf16x2_hw));
}

__device__ __forceinline__ uint32_t f32_to_bf16(float f) { return pack_bf16x2(f, 0.f) & 0xffffu; }

// Activation access: T is float (fp32) or bf16_t (bf16 bits).
template <typename T>
struct Act;

template <>
struct Act<float> {
  static constexpr int kVec = 4;  // elements per 16-byte vector
  __device__ static __forceinline__ float load(const float* p) { return *p; }
  __device__ static __forceinline__ void store(float* p, float v) { *p = v; }
  __device__ static __forceinline__ void unpack(const uint4& v, float* f) {
    f[0] = __uint_as_float(v.x);
    f[1] = __uint_as_float(v.y);
    f[2] = __uint_as_float(v.z);
    f[3] = __uint_as_float(v.w);
  }
  __device__ static __forceinline__ uint4 pack(const float* f) {
    return make_uint4(__float_as_uint(f[0]), __float_as_uint(f[1]), __float_as_uint(f[2]),
                      __float_as_uint(f[3]));
  }
};

template <>
struct Act<bf16_t> {
  static constexpr int kVec = 8;
  __device__ static __forceinline__ float load(const bf16_t* p) { return bf16_to_f32(*p); }
  __device__ static __forceinline__ void store(bf16_t* p, float v) { *p = (bf16_t)f32_to_bf16(v); }
  __device__ static __forceinline__ void unpack(const uint4& v, float* f) {
    const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      f[2 * i] = __uint_as_float(w[i] << 16);
      f[2 * i + 1] = __uint_as_float(w[i] & 0xffff0000u);
    }
  }
  __device__ static __forceinline__ uint4 pack(const float* f) {
    return make_uint4(pack_bf16x2(f[0], f[1]), pack_bf16x2(f[2], f[3]), pack_bf16x2(f[4], f[5]),
                      pack_bf16x2(f[6], f[7]));
  }
};

// ------------------------------------------------------------------ math

// log(1 + e) for e >= 0 from the hardware log: with u = fl(1 + e), log(u) * e / (u - 1)
// cancels the rounding of u (D. Goldberg, "What every computer scientist should know about
// floating-point arithmetic", 1991, Theorem 4); a few ulp.
__device__ __forceinline__ float log1p_pos(float e) {
  const float u = 1.f + e;
  return u == 1.f ? e : __logf(u) * (e * __builtin_amdgcn_rcpf(u - 1.f));
}

// softplus without a clamp; above 20 the identity is exact to fp32 precision.
__device__ __forceinline__ float softplus_f32(float v) { return v > 20.f ? v : log1p_pos(__expf(v)); }

// silu(v) = v / (1 + e^-v); the reciprocal is the hardware approximation (~1 ulp), far
// below the bf16 / fp32 output rounding of every op that uses it.
__device__ __forceinline__ float silu_f32(float v) { return v * __builtin_amdgcn_rcpf(1.f + __expf(-v)); }

// Sum over aligned groups of q lanes (q a power of two <= 64, uniform), every lane of a
// group receiving the group's sum.  Within rows of 16 lanes the partners come from DPP
// (quad permutes, then the half-row and row mirrors: after each step all lanes of the
// growing group hold the same partial sum), across rows from a swizzle (xor 16) and a
// permute (xor 32), so most steps cost no LDS round trip.
__device__ __forceinline__ float group_sum(float v, int q) {
  if (q >= 2) v += __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), 0xB1, 0xF, 0xF, false));
  if (q >= 4) v += __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), 0x4E, 0xF, 0xF, false));
  if (q >= 8) v += __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), 0x141, 0xF, 0xF, false));
  if (q >= 16) v += __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), 0x140, 0xF, 0xF, false));
  if (q >= 32) v += __int_as_float(__builtin_amdgcn_ds_swizzle(__float_as_int(v), 0x401F));
  if (q >= 64) v += __shfl_xor(v, 32, 64);
  return v;
}

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v += __shfl_xor(v, o, 64);
  return v;
}

// Batches of at most this many sequences get their sequence and segment tables from the first
// launch that reads them (one launch fewer); larger ones from the segment-table kernel.
constexpr int kTableSeqs = 256;

// Segment `seg` of a batch of S <= kThreads sequences (row offsets cu[0..S]) cut into segments
// of L rows aligned to each sequence's first row, the sequences' segments numbered in order:
// (sequence, first row, rows, index in its sequence), as the segment-table kernel writes it;
// an empty segment when no sequence has one of that number.  One thread per sequence, every
// thread of the kThreads-thread workgroup taking part (two barriers); with `write` the
// workgroup also stores both tables (seq_info: first segment, segments).
template <int kThreads>
__device__ int4 own_segment(const int32_t* __restrict__ cu, int S, int L, int seg, int2* __restrict__ seq_info,
                            int4* __restrict__ seg_info, bool write) {
  static_assert(kThreads % 64 == 0 && kThreads <= 1024, "whole waves");
  __shared__ int wsum[kThreads / 64];
  __shared__ int4 found;
  const int t = threadIdx.x, lane = t & 63, w = t >> 6;
  int c0 = 0, len = 0, n = 0;
  if (t < S) {
    c0 = cu[t];
    len = cu[t + 1] - c0;
    n = (len + L - 1) / L;
  }
  int incl = n;  // inclusive prefix sum of the segment counts over the sequences
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const int v = __shfl_up(incl, o);
    if (lane >= o) incl += v;
  }
  if (lane == 63) wsum[w] = incl;
  if (t == 0) found = make_int4(0, 0, 0, 0);
  __syncthreads();
  for (int i = 0; i < w; ++i) incl += wsum[i];
  const int first = incl - n;
  if (t < S && seg >= first && seg < first + n) {
    const int k = seg - first;
    found = make_int4(t, c0 + k * L, min(L, len - k * L), k);
  }
  if (write && t < S) {
    seq_info[t] = make_int2(first, n);
    for (int k = 0; k < n; ++k) seg_info[first + k] = make_int4(t, c0 + k * L, min(L, len - k * L), k);
  }
  __syncthreads();
  return found;
}

// ------------------------------------------------------- chunked scan workspace
//
// Sequences are cut into segments of at most seg_len rows (aligned to each
// sequence's first row).  Layout (each section 256-byte aligned):
//   seq_info  int2  [S]        (first segment index, number of segments)
//   seg_info  int4  [nseg]     (sequence, first row, rows, index within sequence)
//   seg_decay f32   [nseg][H]  exp(sum of log-decays over the segment), 0 when that sum is
//                              below -60 (the carried state is dropped)
//   seg_start i32   [nseg][H]  MFMA path: the first chunk of the segment's local-state walk,
//                              with a flag where that walk is left to the next segment's
//                              output kernel (the state is then not stored)
//   seg_chunk f32   [nseg][64][H]  MFMA path: log-decay sums of the segment's chunks
//   seg_state f32   [nseg][H][P][N]  at the index of segment k + 1: the local end state
//                                    of segment k, then the state entering segment k + 1;
//                                    at a sequence's first index, a copy of its slot
//                                    (resumed sequences of several segments only)
struct ScanLayout {
  int64_t nseg;
  int32_t seg_len;
  size_t off_seq_info, off_seg_info, off_seg_decay, off_seg_start, off_seg_chunk, off_seg_state, total;
};

ScanLayout scan_layout(const mamba2_recurrent_batch* rb, const mamba2_dims* d, int32_t seg_len);
int32_t scan_segment_length(const mamba2_recurrent_batch* rb, const mamba2_dims* d, bool mfma);
bool scan_uses_mfma(const mamba2_dims* d);

// ------------------------------------------------------------------ launchers
// Each returns hipSuccess or the launch error.  Shapes are validated by the caller.

struct BatchDev {
  const int32_t* cu_seqlens;  // [S+1]
  const int32_t* slots;       // [S]
  const uint8_t* fresh;       // [S]
  int32_t num_seqs;
  int32_t num_rows;
};

hipError_t launch_conv1d(void* dst, const void* x, const float* w, const float* b, void* conv_state,
                         const BatchDev& bd, int32_t Dc, int32_t K, int32_t act, hipStream_t st);

hipError_t launch_gated_rmsnorm(void* dst, const void* x, const void* z, const float* w,
                                int32_t groups, float eps, int32_t rows, int32_t Di, int32_t act,
                                hipStream_t st);

hipError_t launch_scan_decode(void* dst, const void* xbc, const void* dt, const float* a_log,
                              const float* dt_bias, const float* D, float* ssm_state,
                              const BatchDev& bd, const mamba2_dims& dims, hipStream_t st);

struct ScanArgs {
  void* y;
  const void* xbc;
  const void* dt;
  const float* a_log;
  const float* dt_bias;
  const float* D;
  float* ssm_state;
  BatchDev bd;
  mamba2_dims dims;
  ScanLayout lay;
  char* ws;
  // every segment's entering state must be left in seg_state (read afterwards, e.g. for
  // snapshots): no local-state walk may be left to the output kernels
  bool keep_seg_states;
  // snapshots written by the MFMA path's output kernel (null: none): the state entering each
  // segment that starts at a positive multiple of snap_every rows of its sequence, packed
  // sequence after sequence as [count][H][P][N]
  float* snaps;
  int32_t snap_every;
};

hipError_t launch_scan_prefill(const ScanArgs& a, hipStream_t st);
hipError_t launch_scan_setup(const ScanArgs& a, hipStream_t st);  // sequence and segment tables
hipError_t launch_scan_pass(const ScanArgs& a, hipStream_t st);
bool decode_supported(const mamba2_dims& dm);
bool decode_grid_fits(const mamba2_dims& dm, int32_t num_seqs);

// ------------------------------------------------------- snapshots and rollback
// Boundaries E, 2E, ... strictly inside each run; packed sequence after sequence.
constexpr int32_t kMaxVerifyRows = 16;
int64_t snapshot_count(const mamba2_recurrent_batch* rb, int32_t E);
int32_t snapshot_max_per_seq(const mamba2_recurrent_batch* rb, int32_t E);
size_t verify_lds_bytes(const mamba2_dims& dm, int32_t max_rows);
hipError_t launch_scan_verify(void* y, const void* xbc, const void* dt, const float* a_log,
                              const float* dt_bias, const float* D, float* pool, float* snaps,
                              const BatchDev& bd, const mamba2_dims& dm, int32_t max_rows, hipStream_t st);
hipError_t launch_conv_snapshots(void* snaps, const void* x, const void* conv_state, const BatchDev& bd,
                                 int32_t maxj, int32_t Dc, int32_t K, int32_t E, int32_t act, hipStream_t st);
hipError_t launch_ssm_snapshots(const ScanArgs& a, float* snaps, int32_t maxj, int32_t E, hipStream_t st);
hipError_t launch_commit(float* ssm_state, void* conv_state, const float* ssm_snaps, const void* conv_snaps,
                         const int32_t* accepted, const BatchDev& bd, const mamba2_dims& dm, int32_t E,
                         hipStream_t st);
// Segment length of the chunked scan when every multiple of E must start a segment
// (0: E is not a multiple of the path's segment unit).
int32_t scan_segment_length_snap(const mamba2_recurrent_batch* rb, const mamba2_dims* d, int32_t E);

// ------------------------------------------------------------------ projections
bool linear_supported(int64_t M, int64_t N, int64_t K, int32_t act);
hipError_t launch_linear(void* dst, const void* x, const void* w, int64_t M, int64_t N, int64_t K, hipStream_t st);

// ------------------------------------------------------------------ padded batches
// pack: dst[T][row] <- real rows of src[B][Lmax][row]; unpack: the reverse, zeros on padding.
hipError_t launch_padded(bool pack, void* dst, const void* src, const BatchDev& bd, int32_t Lmax, int32_t left,
                         int64_t row_bytes, hipStream_t st);

// ------------------------------------------------------------------ timing
// When enabled, kernel launches are bracketed by event records.
void timing_before(hipStream_t st, const char* name);
void timing_after(hipStream_t st);

}  // namespace m2

// Launch a kernel with optional timing and return the launch status.
#define M2_LAUNCH(name, kernel, grid, block, shmem, stream, ...)                 \
  do {                                                                          \
    ::m2::timing_before((stream), (name));                                      \
    hipLaunchKernelGGL((kernel), (grid), (block), (shmem), (stream), __VA_ARGS__); \
    ::m2::timing_after((stream));                                               \
    hipError_t _e = hipGetLastError();                                          \
    if (_e != hipSuccess) return _e;                                            \
  } while (0)
