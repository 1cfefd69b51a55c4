// Chunked selective scan, VALU form (fp32 or bf16 activations, any P and N).
//
// This is the fp32 path and the path for shapes the MFMA kernels do not cover.  A
// segment here is one chunk of at most 64 rows.  Inside a chunk the outputs come
// from the quadratic form of the recurrence; with cs_i = sum_{t<=i} a_t,
// a_t = -exp(A_log) * dt'_t:
//   y_i = sum_{j<=i} (C_i . B_j) exp(cs_i - cs_j) dt'_j x_j + exp(cs_i) C_i . S_in + D x_i,
//   S_out = exp(cs_last) S_in + sum_j exp(cs_last - cs_j) dt'_j x_j (x) B_j,
// which is the per-token recurrence of "feat(backend): Mamba2 ops, with CPU reference
// implementations" (section "Ops", SSMScan) summed in closed form over the chunk.
#include "common.h"

namespace m2 {
namespace {

constexpr int kQ = 64;  // rows per chunk, at most

struct ScanPtrs {
  const int2* seq_info;
  const int4* seg_info;
  float* seg_decay;
  float* seg_state;
};

template <typename T>
__device__ void chunk_prologue(const T* __restrict__ dt, const float* __restrict__ a_log,
                               const float* __restrict__ dt_bias, int row0, int rows, int H, int h,
                               float* dtp, float* cs, float* W, float* total) {
  const int tid = threadIdx.x;
  if (tid < rows) {
    const float v = Act<T>::load(dt + (size_t)(row0 + tid) * H + h) + dt_bias[h];
    dtp[tid] = softplus_f32(v);
  }
  __syncthreads();
  if (tid == 0) {
    const float A = __expf(a_log[h]);
    float c = 0.f;
    for (int j = 0; j < rows; ++j) {
      c += -A * dtp[j];
      cs[j] = c;
    }
    float suf = 0.f;  // sum of a_t over t > j
    for (int j = rows - 1; j >= 0; --j) {
      W[j] = __expf(suf) * dtp[j];
      suf += -A * dtp[j];
    }
    *total = suf;
  }
  __syncthreads();
}

// Local end state of every segment except a sequence's last, stored at the index of the
// next segment (the state that segment starts from, once the pass has run).
template <typename T>
__global__ __launch_bounds__(256) void ssd_generic_state_kernel(
    const T* __restrict__ xbc, const T* __restrict__ dt, const float* __restrict__ a_log,
    const float* __restrict__ dt_bias, ScanPtrs sp, int H, int P, int N, int G) {
  const int seg = blockIdx.x;
  const int h = blockIdx.y;
  const int4 si = sp.seg_info[seg];
  const int2 qi = sp.seq_info[si.x];
  if (si.w == qi.y - 1) return;
  __shared__ float dtp[kQ], cs[kQ], W[kQ], total;
  const int row0 = si.y, rows = si.z;
  chunk_prologue<T>(dt, a_log, dt_bias, row0, rows, H, h, dtp, cs, W, &total);
  const int Di = H * P;
  const size_t Dc = (size_t)Di + 2 * (size_t)G * N;
  const int g = h / (H / G);
  float* out = sp.seg_state + ((size_t)(seg + 1) * H + h) * (size_t)P * N;
  for (int e = threadIdx.x; e < P * N; e += blockDim.x) {
    const int p = e / N, n = e % N;
    float acc = 0.f;
    for (int j = 0; j < rows; ++j) {
      const T* r = xbc + (size_t)(row0 + j) * Dc;
      acc = fmaf(W[j] * Act<T>::load(r + (size_t)h * P + p), Act<T>::load(r + Di + (size_t)g * N + n), acc);
    }
    out[e] = acc;
  }
  if (threadIdx.x == 0) sp.seg_decay[(size_t)seg * H + h] = __expf(total);
}

template <typename T>
__global__ __launch_bounds__(256) void ssd_generic_scan_kernel(
    T* __restrict__ y, const T* __restrict__ xbc, const T* __restrict__ dt,
    const float* __restrict__ a_log, const float* __restrict__ dt_bias,
    const float* __restrict__ Dp, float* __restrict__ pool, const int32_t* __restrict__ slots,
    const uint8_t* __restrict__ fresh, ScanPtrs sp, int H, int P, int N, int G) {
  const int seg = blockIdx.x;
  const int h = blockIdx.y;
  const int4 si = sp.seg_info[seg];
  const int2 qi = sp.seq_info[si.x];
  const bool last = si.w == qi.y - 1;
  __shared__ float dtp[kQ], cs[kQ], W[kQ], total;
  __shared__ float CB[kQ * kQ];
  const int row0 = si.y, rows = si.z;
  chunk_prologue<T>(dt, a_log, dt_bias, row0, rows, H, h, dtp, cs, W, &total);
  const int Di = H * P;
  const size_t Dc = (size_t)Di + 2 * (size_t)G * N;
  const int g = h / (H / G);
  const size_t boff = (size_t)Di + (size_t)g * N;
  const size_t coff = (size_t)Di + (size_t)G * N + (size_t)g * N;
  for (int e = threadIdx.x; e < rows * rows; e += blockDim.x) {
    const int i = e / rows, j = e % rows;
    if (j > i) continue;
    const T* ci = xbc + (size_t)(row0 + i) * Dc + coff;
    const T* bj = xbc + (size_t)(row0 + j) * Dc + boff;
    float acc = 0.f;
    for (int n = 0; n < N; ++n) acc = fmaf(Act<T>::load(ci + n), Act<T>::load(bj + n), acc);
    CB[i * kQ + j] = acc;
  }
  __syncthreads();
  // the state entering the segment: zero for a fresh sequence's first segment; the slot
  // itself for a resumed sequence of one segment (this workgroup alone reads and then
  // writes it); else what the pass left at this segment's index
  const float* Sin = (si.w == 0 && fresh[si.x]) ? nullptr
                     : (si.w == 0 && last) ? pool + ((size_t)slots[si.x] * H + h) * (size_t)P * N
                                           : sp.seg_state + ((size_t)seg * H + h) * (size_t)P * N;
  const float Dh = Dp[h];
  for (int e = threadIdx.x; e < rows * P; e += blockDim.x) {
    const int i = e / P, p = e % P;
    float acc = 0.f;
    for (int j = 0; j <= i; ++j)
      acc = fmaf(CB[i * kQ + j] * __expf(cs[i] - cs[j]) * dtp[j],
                 Act<T>::load(xbc + (size_t)(row0 + j) * Dc + (size_t)h * P + p), acc);
    const T* ci = xbc + (size_t)(row0 + i) * Dc + coff;
    float off = 0.f;
    if (Sin)
      for (int n = 0; n < N; ++n) off = fmaf(Act<T>::load(ci + n), Sin[(size_t)p * N + n], off);
    const float xi = Act<T>::load(xbc + (size_t)(row0 + i) * Dc + (size_t)h * P + p);
    Act<T>::store(y + (size_t)(row0 + i) * Di + (size_t)h * P + p,
                  acc + __expf(cs[i]) * off + Dh * xi);
  }
  __syncthreads();  // every read of Sin (possibly the slot itself) done before the slot is written
  if (last) {
    const float dlast = __expf(cs[rows - 1]);
    float* dstate = pool + ((size_t)slots[si.x] * H + h) * (size_t)P * N;
    for (int e = threadIdx.x; e < P * N; e += blockDim.x) {
      const int p = e / N, n = e % N;
      float acc = Sin ? dlast * Sin[e] : 0.f;
      for (int j = 0; j < rows; ++j) {
        const T* r = xbc + (size_t)(row0 + j) * Dc;
        acc = fmaf(W[j] * Act<T>::load(r + (size_t)h * P + p), Act<T>::load(r + boff + n), acc);
      }
      dstate[e] = acc;
    }
  }
}

template <typename T>
hipError_t launch_t(const ScanArgs& a, hipStream_t st) {
  const ScanPtrs sp{(const int2*)(a.ws + a.lay.off_seq_info), (const int4*)(a.ws + a.lay.off_seg_info),
                    (float*)(a.ws + a.lay.off_seg_decay), (float*)(a.ws + a.lay.off_seg_state)};
  const mamba2_dims& d = a.dims;
  const dim3 grid((unsigned)a.lay.nseg, (unsigned)d.nheads);
  M2_LAUNCH("ssd_generic_state", ssd_generic_state_kernel<T>, grid, dim3(256), 0, st,
            (const T*)a.xbc, (const T*)a.dt, a.a_log, a.dt_bias, sp, d.nheads, d.headdim,
            d.d_state, d.ngroups);
  hipError_t e = launch_scan_pass(a, st);
  if (e != hipSuccess) return e;
  M2_LAUNCH("ssd_generic_scan", ssd_generic_scan_kernel<T>, grid, dim3(256), 0, st, (T*)a.y,
            (const T*)a.xbc, (const T*)a.dt, a.a_log, a.dt_bias, a.D, a.ssm_state, a.bd.slots, a.bd.fresh, sp,
            d.nheads, d.headdim, d.d_state, d.ngroups);
  return hipSuccess;
}

}  // namespace

hipError_t launch_scan_generic(const ScanArgs& a, hipStream_t st) {
  if (a.dims.act_dtype == MAMBA2_DTYPE_BF16) return launch_t<bf16_t>(a, st);
  return launch_t<float>(a, st);
}

}  // namespace m2
