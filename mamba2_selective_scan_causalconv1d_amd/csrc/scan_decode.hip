// One-row decode step of the selective scan for gfx950.
//
// Operation ("feat(backend): Mamba2 ops, with CPU reference implementations", section
// "Ops", SSMScan, with one row per sequence): dt' = softplus(dt + dt_bias),
//   h[p, n] <- h[p, n] * exp(-exp(A_log) * dt') + (dt' * x[p]) * B[n],
//   y[p] = sum_n h[p, n] * C[n] + D * x[p],
// head h reading B and C of group h / (H / G); a fresh sequence starts from zero and
// never reads its slot.
//
// Mapping: the head's fp32 state [P][N] is cut into blocks of whole rows, one
// workgroup per (sequence, head, block); for P = 64, N = 128 a block is 16 rows
// (8 KiB), two float4s per thread.  The state is streamed once in and once out with
// 16-byte non-temporal accesses (it is not reused within the step, and keeping it out
// of the caches leaves them to the step's small operands); consecutive threads take
// consecutive float4s.  A thread keeps the same four state columns for every row it
// visits, so its B and C values are loaded once; the row sums of h * C are reduced
// over the N/4 lanes that share a row.  Small blocks with few loads per thread keep
// many workgroups in flight, which is what this HBM-streaming kernel (~0.75 flop per
// byte) needs.
#include "common.h"

namespace m2 {
namespace {

typedef float f4v __attribute__((ext_vector_type(4)));

template <typename T>
__device__ __forceinline__ void load4(const T* p, float* f);

template <>
__device__ __forceinline__ void load4<float>(const float* p, float* f) {
  const float4 v = *reinterpret_cast<const float4*>(p);
  f[0] = v.x;
  f[1] = v.y;
  f[2] = v.z;
  f[3] = v.w;
}

template <>
__device__ __forceinline__ void load4<bf16_t>(const bf16_t* p, float* f) {
  const uint2 v = *reinterpret_cast<const uint2*>(p);
  f[0] = bf16_to_f32(v.x & 0xffffu);
  f[1] = bf16_to_f32(v.x >> 16);
  f[2] = bf16_to_f32(v.y & 0xffffu);
  f[3] = bf16_to_f32(v.y >> 16);
}

// KP float4s per thread; the launch's S * H * nblk workgroups each cover KP * blockDim.x
// float4s (one block) of one head's state of one sequence.  Workgroup b runs on XCD b % 8,
// and each XCD takes a contiguous run of (sequence, head, block) items, so a sequence's
// row is fetched into one XCD's L2 and each XCD streams whole slots in address order (on the
// 256-request decode step: 136.9 -> 133.6 us against consecutive items dealt round robin).
// 2^lq4 = N / 4 lanes share a state row (a power of two dividing 64); hpg heads per group.
// The slot index and the fresh flag are buffer loads issued together with the row's loads
// (as scalar loads, which miss the scalar cache on every new sequence, the kernel took 2 us
// longer).
template <typename T, int KP>
__global__ __launch_bounds__(256) void scan_decode_kernel(
    T* __restrict__ y, const T* __restrict__ xbc, const T* __restrict__ dt,
    const float* __restrict__ a_log, const float* __restrict__ dt_bias,
    const float* __restrict__ Dp, float* __restrict__ pool, const int32_t* __restrict__ slots,
    const uint8_t* __restrict__ fresh, int S, int H, int P, int N, int G, int hpg, int lq4, int nblk) {
  const int J = H * nblk;
  const int nitems = S * J;
  const int b = blockIdx.x, xcd = b & 7;
  const int item = xcd * (nitems >> 3) + min(xcd, nitems & 7) + (b >> 3);
  const int r = item / J;
  const int hb = item - r * J;
  const int h = hb / nblk;
  const int blk = hb - h * nblk;
  const int tid = threadIdx.x;
  const int nthr = blockDim.x;
  const int Q4 = 1 << lq4;
  const int Di = H * P;
  const size_t Dc = (size_t)Di + 2 * (size_t)G * N;
  const int g = G == 1 ? 0 : h / hpg;
  const int f0 = blk * KP * nthr;  // first float4 of the block within the head
  const int n0 = 4 * (tid & (Q4 - 1));
  const float bias = dt_bias[h];
  const float A = __expf(a_log[h]);
  const float d = Dp[h];
  const T* row = xbc + (size_t)r * Dc;
  typedef __amdgpu_buffer_rsrc_t Rsrc;
  const Rsrc rs = __builtin_amdgcn_make_buffer_rsrc(const_cast<int32_t*>(slots + r), 0, 4, 0x00020000);
  const Rsrc rf = __builtin_amdgcn_make_buffer_rsrc(const_cast<uint8_t*>(fresh + r), 0, 1, 0x00020000);
  const uint32_t is_fresh = __builtin_amdgcn_raw_buffer_load_b8(rf, 0, 0, 0);
  const int slot = __builtin_amdgcn_raw_buffer_load_b32(rs, 0, 0, 0);
  f4v* st = reinterpret_cast<f4v*>(pool + ((size_t)slot * H + h) * (size_t)P * N) + f0;
  f4v hv[KP];
  if (is_fresh) {
#pragma unroll
    for (int k = 0; k < KP; ++k) hv[k] = f4v{0.f, 0.f, 0.f, 0.f};
  } else {
#pragma unroll
    for (int k = 0; k < KP; ++k) hv[k] = __builtin_nontemporal_load(st + k * nthr + tid);
  }
  const float v = Act<T>::load(dt + (size_t)r * H + h) + bias;
  float Bv[4], Cv[4];
  load4<T>(row + Di + (size_t)g * N + n0, Bv);
  load4<T>(row + Di + (size_t)G * N + (size_t)g * N + n0, Cv);
  float xs[KP];
#pragma unroll
  for (int k = 0; k < KP; ++k) xs[k] = Act<T>::load(row + (size_t)h * P + ((f0 + k * nthr + tid) >> lq4));
  const float dtp = softplus_f32(v);
  const float dA = __expf(-A * dtp);
  float part[KP];
#pragma unroll
  for (int k = 0; k < KP; ++k) {
    const float c = dtp * xs[k];
    f4v s = hv[k];
    s.x = fmaf(c, Bv[0], s.x * dA);
    s.y = fmaf(c, Bv[1], s.y * dA);
    s.z = fmaf(c, Bv[2], s.z * dA);
    s.w = fmaf(c, Bv[3], s.w * dA);
    hv[k] = s;
    part[k] = fmaf(s.x, Cv[0], fmaf(s.y, Cv[1], fmaf(s.z, Cv[2], s.w * Cv[3])));
  }
#pragma unroll
  for (int k = 0; k < KP; ++k) __builtin_nontemporal_store(hv[k], st + k * nthr + tid);
#pragma unroll
  for (int k = 0; k < KP; ++k) part[k] = group_sum(part[k], Q4);
  if ((tid & (Q4 - 1)) == 0) {
#pragma unroll
    for (int k = 0; k < KP; ++k) {
      const int p = (f0 + k * nthr + tid) >> lq4;
      Act<T>::store(y + (size_t)r * Di + (size_t)h * P + p, fmaf(d, xs[k], part[k]));
    }
  }
}

// A short run per sequence (1..kMaxVerifyRows rows, e.g. a speculative draft), in the
// decode mapping: the block's state stays in registers over the run's rows, so it is read
// and written once whatever the run length.  The run's B, C, x (the block's rows) and
// per-row decay scalars are first staged in LDS ([L][2N + rb] and [L][2]), then the rows
// are applied in order with the arithmetic of the one-row kernel (a run of one row gives
// its results bit for bit).  snaps (may be null): the state after every row but the last,
// [T - S][H][P][N], sequence r's first at row offset cu[r] - r.
template <typename T, int KP>
__global__ __launch_bounds__(256) void scan_verify_kernel(
    T* __restrict__ y, const T* __restrict__ xbc, const T* __restrict__ dt,
    const float* __restrict__ a_log, const float* __restrict__ dt_bias,
    const float* __restrict__ Dp, float* __restrict__ pool, float* __restrict__ snaps,
    const int32_t* __restrict__ cu, const int32_t* __restrict__ slots, const uint8_t* __restrict__ fresh,
    int S, int H, int P, int N, int G, int nblk) {
  extern __shared__ float lds[];
  // (sequence, head, block) items in XCD-contiguous order, as in the one-row kernel
  const int J = H * nblk;
  const int nitems = S * J;
  const int b = blockIdx.x, xcd = b & 7;
  const int item = xcd * (nitems >> 3) + min(xcd, nitems & 7) + (b >> 3);
  const int r = item / J;
  const int hb = item - r * J;
  const int h = hb / nblk;
  const int blk = hb - h * nblk;
  const int tid = threadIdx.x;
  const int nthr = blockDim.x;
  const int Q4 = N >> 2;
  const int Di = H * P;
  const size_t Dc = (size_t)Di + 2 * (size_t)G * N;
  const int g = h / (H / G);
  const int f0 = blk * KP * nthr;
  const int row0 = cu[r];
  const int L = cu[r + 1] - row0;

  const int rb = KP * nthr / Q4;
  const int pfirst = f0 / Q4;
  const int W = 2 * N + rb;
  float* sw = lds;           // [L][W]: B, C, the block's x
  float* sdt = lds + L * W;  // [L][2]: dt', exp(-exp(A_log) dt')
  // The state goes out first, then the staging loads (eight per thread and pass, indices
  // clamped into the run so that every load is unconditional) and the dt values: the
  // workgroup pays one trip to memory for all of them.
  const int cB = Di + g * N, cC = Di + (G + g) * N, cX = h * P + pfirst;
  const int nst = L * W;
  auto stage_load = [&](int i0, float* v) {
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const int i = min(i0 + u * nthr, nst - 1);
      const int t = i / W;
      const int c = i - t * W;
      const int ch = c < N ? cB + c : (c < 2 * N ? cC + (c - N) : cX + (c - 2 * N));
      v[u] = Act<T>::load(xbc + (size_t)(row0 + t) * Dc + ch);
    }
  };
  auto stage_store = [&](int i0, const float* v) {
#pragma unroll
    for (int u = 0; u < 8; ++u)
      if (i0 + u * nthr < nst) sw[i0 + u * nthr] = v[u];
  };

  f4v* st = reinterpret_cast<f4v*>(pool + ((size_t)slots[r] * H + h) * (size_t)P * N) + f0;
  f4v hv[KP];
  if (fresh[r]) {
#pragma unroll
    for (int k = 0; k < KP; ++k) hv[k] = f4v{0.f, 0.f, 0.f, 0.f};
  } else {
#pragma unroll
    for (int k = 0; k < KP; ++k) hv[k] = __builtin_nontemporal_load(st + k * nthr + tid);
  }
  float v0[8];
  stage_load(tid, v0);
  const float dtv = Act<T>::load(dt + (size_t)(row0 + min(tid, L - 1)) * H + h);
  const float bias = dt_bias[h];
  const float A = __expf(a_log[h]);

  stage_store(tid, v0);
  if (tid < L) {
    const float dtp = softplus_f32(dtv + bias);
    sdt[2 * tid] = dtp;
    sdt[2 * tid + 1] = __expf(-A * dtp);
  }
  for (int i0 = tid + 8 * nthr; i0 < nst; i0 += 8 * nthr) {  // runs of 8 rows and more (W <= 2 nthr)
    float v[8];
    stage_load(i0, v);
    stage_store(i0, v);
  }
  __syncthreads();

  const int n0 = 4 * (tid % Q4);
  const float d = Dp[h];
  const size_t hpn = (size_t)H * P * N;
  f4v* snap0 = snaps ? reinterpret_cast<f4v*>(snaps + (size_t)(row0 - r) * hpn + (size_t)h * P * N) + f0
                     : nullptr;
  for (int t = 0; t < L; ++t) {
    const float* rw = sw + t * W;
    const float dtp = sdt[2 * t];
    const float dA = sdt[2 * t + 1];
    const float Bv[4] = {rw[n0], rw[n0 + 1], rw[n0 + 2], rw[n0 + 3]};
    const float Cv[4] = {rw[N + n0], rw[N + n0 + 1], rw[N + n0 + 2], rw[N + n0 + 3]};
    float part[KP], xs[KP];
#pragma unroll
    for (int k = 0; k < KP; ++k) {
      xs[k] = rw[2 * N + (f0 + k * nthr + tid) / Q4 - pfirst];
      const float c = dtp * xs[k];
      f4v s = hv[k];
      s.x = fmaf(c, Bv[0], s.x * dA);
      s.y = fmaf(c, Bv[1], s.y * dA);
      s.z = fmaf(c, Bv[2], s.z * dA);
      s.w = fmaf(c, Bv[3], s.w * dA);
      hv[k] = s;
      part[k] = fmaf(s.x, Cv[0], fmaf(s.y, Cv[1], fmaf(s.z, Cv[2], s.w * Cv[3])));
    }
    if (snap0 && t + 1 < L) {
#pragma unroll
      for (int k = 0; k < KP; ++k) snap0[(size_t)t * (hpn / 4) + k * nthr + tid] = hv[k];
    }
#pragma unroll
    for (int k = 0; k < KP; ++k) part[k] = group_sum(part[k], Q4);
    if ((tid % Q4) == 0) {
#pragma unroll
      for (int k = 0; k < KP; ++k) {
        const int p = (f0 + k * nthr + tid) / Q4;
        Act<T>::store(y + (size_t)(row0 + t) * Di + (size_t)h * P + p, fmaf(d, xs[k], part[k]));
      }
    }
  }
#pragma unroll
  for (int k = 0; k < KP; ++k) __builtin_nontemporal_store(hv[k], st + k * nthr + tid);
}

// Block shape: 512 float4s (two per thread) when the head's state is a multiple of
// that, else the whole head in one workgroup (f4 = 256: one per thread; f4 < 256: f4
// threads, one each).
struct DecodeShape {
  int nthr, kp, nblk;
};

DecodeShape decode_shape(const mamba2_dims& dm) {
  const int64_t f4 = (int64_t)dm.headdim * (dm.d_state / 4);  // float4s per head state
  if (f4 % 512 == 0) return DecodeShape{256, 2, (int)(f4 / 512)};
  return DecodeShape{(int)f4, 1, 1};
}

// The one-row decode kernel's blocks: 256 float4s (two per thread of 128) when the head's
// state is a multiple of that (on the 256-request decode step, with the XCD-contiguous
// order: 134.3 us against 135.1 us for 512-float4 blocks and 140.4 us for four float4s per
// thread), else the whole head.
DecodeShape decode_step_shape(const mamba2_dims& dm) {
  const int64_t f4 = (int64_t)dm.headdim * (dm.d_state / 4);
  if (f4 % 256 == 0) return DecodeShape{128, 2, (int)(f4 / 256)};
  return DecodeShape{(int)f4, 1, 1};
}

template <typename T>
hipError_t launch_t(void* y, const void* xbc, const void* dt, const float* a_log,
                    const float* dt_bias, const float* D, float* pool, const BatchDev& bd,
                    const mamba2_dims& dm, hipStream_t st) {
  const DecodeShape sh = decode_step_shape(dm);
  const dim3 grid((unsigned)((int64_t)bd.num_seqs * dm.nheads * sh.nblk));
  int lq4 = 0;
  while ((1 << lq4) < dm.d_state / 4) ++lq4;
  const int hpg = dm.nheads / dm.ngroups;
  if (sh.kp == 2) {
    M2_LAUNCH("scan_decode", (scan_decode_kernel<T, 2>), grid, dim3(sh.nthr), 0, st, (T*)y, (const T*)xbc,
              (const T*)dt, a_log, dt_bias, D, pool, bd.slots, bd.fresh, bd.num_seqs, dm.nheads, dm.headdim,
              dm.d_state, dm.ngroups, hpg, lq4, sh.nblk);
  } else {
    M2_LAUNCH("scan_decode", (scan_decode_kernel<T, 1>), grid, dim3(sh.nthr), 0, st, (T*)y, (const T*)xbc,
              (const T*)dt, a_log, dt_bias, D, pool, bd.slots, bd.fresh, bd.num_seqs, dm.nheads, dm.headdim,
              dm.d_state, dm.ngroups, hpg, lq4, sh.nblk);
  }
  return hipSuccess;
}

template <typename T>
hipError_t launch_verify_t(void* y, const void* xbc, const void* dt, const float* a_log, const float* dt_bias,
                           const float* D, float* pool, float* snaps, const BatchDev& bd, const mamba2_dims& dm,
                           int32_t max_rows, hipStream_t st) {
  const DecodeShape sh = decode_shape(dm);
  const dim3 grid((unsigned)((int64_t)bd.num_seqs * dm.nheads * sh.nblk));
  const int rb = sh.kp * sh.nthr / (dm.d_state / 4);
  const size_t shmem = (size_t)max_rows * (2 * dm.d_state + rb + 2) * sizeof(float);
  if (sh.kp == 2) {
    M2_LAUNCH("scan_verify", (scan_verify_kernel<T, 2>), grid, dim3(sh.nthr), shmem, st, (T*)y, (const T*)xbc,
              (const T*)dt, a_log, dt_bias, D, pool, snaps, bd.cu_seqlens, bd.slots, bd.fresh, bd.num_seqs, dm.nheads,
              dm.headdim, dm.d_state, dm.ngroups, sh.nblk);
  } else {
    M2_LAUNCH("scan_verify", (scan_verify_kernel<T, 1>), grid, dim3(sh.nthr), shmem, st, (T*)y, (const T*)xbc,
              (const T*)dt, a_log, dt_bias, D, pool, snaps, bd.cu_seqlens, bd.slots, bd.fresh, bd.num_seqs, dm.nheads,
              dm.headdim, dm.d_state, dm.ngroups, sh.nblk);
  }
  return hipSuccess;
}

}  // namespace

// LDS the run staging takes for runs of up to max_rows rows.
size_t verify_lds_bytes(const mamba2_dims& dm, int32_t max_rows) {
  const DecodeShape sh = decode_shape(dm);
  const int rb = sh.kp * sh.nthr / (dm.d_state / 4);
  return (size_t)max_rows * (2 * dm.d_state + rb + 2) * sizeof(float);
}

hipError_t launch_scan_verify(void* y, const void* xbc, const void* dt, const float* a_log,
                              const float* dt_bias, const float* D, float* pool, float* snaps,
                              const BatchDev& bd, const mamba2_dims& dm, int32_t max_rows, hipStream_t st) {
  if (dm.act_dtype == MAMBA2_DTYPE_BF16)
    return launch_verify_t<bf16_t>(y, xbc, dt, a_log, dt_bias, D, pool, snaps, bd, dm, max_rows, st);
  return launch_verify_t<float>(y, xbc, dt, a_log, dt_bias, D, pool, snaps, bd, dm, max_rows, st);
}

// Shapes the decode kernel covers: N % 4 == 0 with N/4 a power of two <= 64 (a state
// row's lanes lie in one wavefront), and P*N/4 float4s per head either a multiple of
// 512, exactly 256, or below 256 and a multiple of 64 (whole wavefronts).
bool decode_supported(const mamba2_dims& dm) {
  const int N = dm.d_state;
  if (N % 4 != 0) return false;
  const int Q4 = N / 4;
  if (Q4 > 64 || (Q4 & (Q4 - 1)) != 0) return false;
  const int64_t f4 = (int64_t)dm.headdim * Q4;
  return f4 % 512 == 0 || f4 == 256 || (f4 < 256 && f4 % 64 == 0);
}

// Both launches are one-dimensional: S * H * blocks workgroups, under 2^32 work-items and
// under 2^31 items.
bool decode_grid_fits(const mamba2_dims& dm, int32_t num_seqs) {
  for (const DecodeShape sh : {decode_shape(dm), decode_step_shape(dm)}) {
    const int64_t items = (int64_t)num_seqs * dm.nheads * sh.nblk;
    if (items * sh.nthr >= ((int64_t)1 << 32) || items >= ((int64_t)1 << 31)) return false;
  }
  return true;
}

hipError_t launch_scan_decode(void* y, const void* xbc, const void* dt, const float* a_log,
                              const float* dt_bias, const float* D, float* pool,
                              const BatchDev& bd, const mamba2_dims& dm, hipStream_t st) {
  if (dm.act_dtype == MAMBA2_DTYPE_BF16)
    return launch_t<bf16_t>(y, xbc, dt, a_log, dt_bias, D, pool, bd, dm, st);
  return launch_t<float>(y, xbc, dt, a_log, dt_bias, D, pool, bd, dm, st);
}

}  // namespace m2
