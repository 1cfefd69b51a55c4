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
//
// Mapping: one 256-thread workgroup per (chunk, head).  Operands are staged in LDS as fp32
// tiles of 64 rows x 64 columns (p, n or chunk-row columns), zero past the chunk, P and N,
// and every contraction is a sum of outer products: per step of its inner index a thread
// reads a float4 of each operand and updates its 4 x 4 block of the 64 x 64 output tile.
// Contractions over n or over the chunk rows read transposed tiles ([k][row]), those over
// chunk rows with x read x tiles as they are ([row][p]).
#include "common.h"

namespace m2 {
namespace {

constexpr int kQ = 64;        // rows per chunk, at most
constexpr int kT = 64;        // tile width
constexpr int kLd = kT + 4;   // tile row pitch (floats): 16-byte aligned rows
constexpr int kThreads = 256;

struct ScanPtrs {
  const int2* seq_info;
  const int4* seg_info;
  float* seg_decay;
  float* seg_state;
};

typedef float Tile[kQ][kLd];

// dt'_j, cs_j and W_j = exp(cs_last - cs_j) dt'_j of the chunk's rows (the first wave, one row
// per lane, cs by a wave prefix sum), and the chunk's total log-decay cs_last.
template <typename T>
__device__ __forceinline__ void chunk_prologue(const T* __restrict__ dt, const float* __restrict__ a_log,
                               const float* __restrict__ dt_bias, int row0, int rows, int H, int h,
                               float* dtp, float* cs, float* W, float* total) {
  const int j = threadIdx.x;
  if (j < 64) {
    float d = 0.f;
    if (j < rows) d = softplus_f32(Act<T>::load(dt + (size_t)(row0 + j) * H + h) + dt_bias[h]);
    float c = -__expf(a_log[h]) * d;  // zero past the chunk's rows
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
      const float u = __shfl_up(c, o, 64);
      if (j >= o) c += u;
    }
    const float last = __shfl(c, 63, 64);
    if (j < rows) {
      dtp[j] = d;
      cs[j] = c;
      W[j] = __expf(last - c) * d;
    }
    if (j == 0) *total = last;
  }
  __syncthreads();
}

// dst[r][c] = src row (row0 + r), column c0 + c (times wr[r] when given); zero past rows or ncol.
template <typename T>
__device__ __forceinline__ void stage_rows(Tile& dst, const T* __restrict__ xbc, size_t Dc, int row0, int rows,
                                           size_t col, int c0, int ncol, const float* wr) {
  for (int e = threadIdx.x; e < kQ * kT; e += kThreads) {
    const int r = e / kT, c = e % kT;
    float v = 0.f;
    if (r < rows && c0 + c < ncol) {
      v = Act<T>::load(xbc + (size_t)(row0 + r) * Dc + col + c0 + c);
      if (wr) v *= wr[r];
    }
    dst[r][c] = v;
  }
}
// dst[c][r] = src row (row0 + r), column c0 + c: the transposed tile.
template <typename T>
__device__ __forceinline__ void stage_cols(Tile& dst, const T* __restrict__ xbc, size_t Dc, int row0, int rows,
                                           size_t col, int c0, int ncol) {
  for (int e = threadIdx.x; e < kQ * kT; e += kThreads) {
    const int r = e / kT, c = e % kT;
    dst[c][r] = (r < rows && c0 + c < ncol) ? Act<T>::load(xbc + (size_t)(row0 + r) * Dc + col + c0 + c) : 0.f;
  }
}

__device__ __forceinline__ float4 f4at(const float* p) { return *reinterpret_cast<const float4*>(p); }

// acc[a][b] += u[a] v[b]
__device__ __forceinline__ void outer4(float (&acc)[4][4], const float4& u, const float4& v) {
  const float uu[4] = {u.x, u.y, u.z, u.w}, vv[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
  for (int a = 0; a < 4; ++a)
#pragma unroll
    for (int b = 0; b < 4; ++b) acc[a][b] = fmaf(uu[a], vv[b], acc[a][b]);
}

// out[p][n] = (Sin ? dlast Sin[p][n] : 0) + sum_j W_j x_j[p] B_j[n], over 64 x 64 tiles of
// (p, n); thread t owns rows p0 + 4 (t / 16).. and columns n0 + 4 (t % 16)..  Sin may be out
// itself (each element is read and then written by the same thread); the first barrier orders
// these writes after every earlier read of the workgroup.
template <typename T>
__device__ __forceinline__ void state_tiles(float* __restrict__ out, const float* Sin, float dlast, const T* __restrict__ xbc,
                            size_t Dc, int row0, int rows, size_t xcol, size_t bcol, int P, int N,
                            const float* W, Tile& sX, Tile& sB) {
  const int tp = threadIdx.x / 16, tn = threadIdx.x % 16;
  for (int p0 = 0; p0 < P; p0 += kT) {
    for (int n0 = 0; n0 < N; n0 += kT) {
      __syncthreads();  // the previous tile's reads (and every earlier read of Sin) are done
      stage_rows<T>(sX, xbc, Dc, row0, rows, xcol, p0, P, W);
      stage_rows<T>(sB, xbc, Dc, row0, rows, bcol, n0, N, nullptr);
      __syncthreads();
      float acc[4][4] = {};
      for (int j = 0; j < rows; ++j) outer4(acc, f4at(&sX[j][4 * tp]), f4at(&sB[j][4 * tn]));
#pragma unroll
      for (int a = 0; a < 4; ++a) {
        const int p = p0 + 4 * tp + a;
        if (p >= P) break;
#pragma unroll
        for (int b = 0; b < 4; ++b) {
          const int n = n0 + 4 * tn + b;
          if (n < N) {
            const size_t e = (size_t)p * N + n;
            out[e] = Sin ? fmaf(dlast, Sin[e], acc[a][b]) : acc[a][b];
          }
        }
      }
    }
  }
}

// Local end state of every segment except a sequence's last, stored at the index of the
// next segment (the state that segment starts from, once the pass has run).
template <typename T>
__global__ __launch_bounds__(kThreads) void ssd_generic_state_kernel(
    const T* __restrict__ xbc, const T* __restrict__ dt, const float* __restrict__ a_log,
    const float* __restrict__ dt_bias, ScanPtrs sp, int H, int P, int N, int G) {
  const int seg = blockIdx.x;
  const int h = blockIdx.y;
  const int4 si = sp.seg_info[seg];
  const int2 qi = sp.seq_info[si.x];
  if (si.w == qi.y - 1) return;  // uniform over the workgroup
  __shared__ float dtp[kQ], cs[kQ], W[kQ], total;
  __shared__ __attribute__((aligned(16))) Tile sX, sB;
  const int row0 = si.y, rows = si.z;
  chunk_prologue<T>(dt, a_log, dt_bias, row0, rows, H, h, dtp, cs, W, &total);
  const int Di = H * P;
  const size_t Dc = (size_t)Di + 2 * (size_t)G * N;
  const int g = h / (H / G);
  float* out = sp.seg_state + ((size_t)(seg + 1) * H + h) * (size_t)P * N;
  state_tiles<T>(out, nullptr, 0.f, xbc, Dc, row0, rows, (size_t)h * P, (size_t)Di + (size_t)g * N, P, N, W,
                 sX, sB);
  if (threadIdx.x == 0) sp.seg_decay[(size_t)seg * H + h] = __expf(total);
}

template <typename T>
__global__ __launch_bounds__(kThreads) void ssd_generic_scan_kernel(
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
  __shared__ __attribute__((aligned(16))) Tile sM, sX, sU, sV;  // M^T [j][i]; x [j][p]; staging
  const int row0 = si.y, rows = si.z;
  chunk_prologue<T>(dt, a_log, dt_bias, row0, rows, H, h, dtp, cs, W, &total);
  const int Di = H * P;
  const size_t Dc = (size_t)Di + 2 * (size_t)G * N;
  const int g = h / (H / G);
  const size_t xcol = (size_t)h * P, bcol = (size_t)Di + (size_t)g * N, ccol = (size_t)Di + (size_t)(G + g) * N;
  const int ti = threadIdx.x / 16, tj = threadIdx.x % 16;  // 4 x 4 output block (rows 4 ti.., columns 4 tj..)

  // M^T[j][i] = (C_i . B_j) exp(cs_i - cs_j) dt'_j for j <= i, else 0: C^T and B^T tiles over n
  {
    float gacc[4][4] = {};
    for (int n0 = 0; n0 < N; n0 += kT) {
      __syncthreads();
      stage_cols<T>(sU, xbc, Dc, row0, rows, ccol, n0, N);
      stage_cols<T>(sV, xbc, Dc, row0, rows, bcol, n0, N);
      __syncthreads();
      if (tj <= ti)
        for (int c = 0; c < kT; ++c) outer4(gacc, f4at(&sU[c][4 * ti]), f4at(&sV[c][4 * tj]));
    }
#pragma unroll
    for (int a = 0; a < 4; ++a) {
      const int i = 4 * ti + a;
#pragma unroll
      for (int b = 0; b < 4; ++b) {
        const int j = 4 * tj + b;
        sM[j][i] = (j <= i && i < rows) ? gacc[a][b] * __expf(cs[i] - cs[j]) * dtp[j] : 0.f;
      }
    }
  }

  // the state entering the segment: zero for a fresh sequence's first segment; the slot
  // itself for a resumed sequence of one segment (this workgroup alone reads and then
  // writes it); else what the pass left at this segment's index
  const float* Sin = (si.w == 0 && fresh[si.x]) ? nullptr
                     : (si.w == 0 && last) ? pool + ((size_t)slots[si.x] * H + h) * (size_t)P * N
                                           : sp.seg_state + ((size_t)seg * H + h) * (size_t)P * N;
  const float Dh = Dp[h];
  // y[i][p] = sum_{j<=i} M[i][j] x_j[p] + exp(cs_i) sum_n C_i[n] Sin[p][n] + D x_i[p], 64-wide p tiles
  for (int p0 = 0; p0 < P; p0 += kT) {
    __syncthreads();  // sM written; the previous tile's reads done
    stage_rows<T>(sX, xbc, Dc, row0, rows, xcol, p0, P, nullptr);
    __syncthreads();
    float dg[4][4] = {}, of[4][4] = {};
    const int jmax = min(rows - 1, 4 * ti + 3);
    for (int j = 0; j <= jmax; ++j) outer4(dg, f4at(&sM[j][4 * ti]), f4at(&sX[j][4 * tj]));
    if (Sin) {
      for (int n0 = 0; n0 < N; n0 += kT) {
        __syncthreads();
        stage_cols<T>(sU, xbc, Dc, row0, rows, ccol, n0, N);
        for (int e = threadIdx.x; e < kT * kT; e += kThreads) {  // sV[c][pp] = Sin[p0 + pp][n0 + c]
          const int pp = e / kT, c = e % kT;
          sV[c][pp] = (p0 + pp < P && n0 + c < N) ? Sin[(size_t)(p0 + pp) * N + n0 + c] : 0.f;
        }
        __syncthreads();
        for (int c = 0; c < kT; ++c) outer4(of, f4at(&sU[c][4 * ti]), f4at(&sV[c][4 * tj]));
      }
    }
#pragma unroll
    for (int a = 0; a < 4; ++a) {
      const int i = 4 * ti + a;
      if (i >= rows) break;
      const float ei = __expf(cs[i]);
#pragma unroll
      for (int b = 0; b < 4; ++b) {
        const int p = p0 + 4 * tj + b;
        if (p < P)
          Act<T>::store(y + (size_t)(row0 + i) * Di + xcol + p, fmaf(ei, of[a][b], fmaf(Dh, sX[i][4 * tj + b], dg[a][b])));
      }
    }
  }
  if (last) {
    float* dstate = pool + ((size_t)slots[si.x] * H + h) * (size_t)P * N;
    state_tiles<T>(dstate, Sin, __expf(total), xbc, Dc, row0, rows, xcol, bcol, P, N, W, sX, sU);
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
