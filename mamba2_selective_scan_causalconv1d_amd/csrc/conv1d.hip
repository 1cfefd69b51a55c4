// Depthwise causal conv1d + SiLU with per-sequence conv-state slots, for gfx950.
//
// Operation ("feat(backend): Mamba2 ops, with CPU reference implementations",
// section "Ops", CausalConv1D): out[t, c] = silu(b[c] + sum_k w[c, k] * win[t + k]),
// win = (K-1 history rows from the slot, or zeros when fresh) ++ the sequence's rows;
// afterwards the slot holds the last K-1 rows of win, bit for bit.
//
// Mapping: one thread owns one 16-byte channel vector (8 bf16 / 4 fp32 channels)
// of a tile of R consecutive packed rows and slides a K-tap window down them in
// registers; a wavefront covers 64 consecutive vectors of a row, so every row
// access is a contiguous 1 KiB.  Input rows are read with non-temporal loads (each
// is read once per launch).  A batch with one row per sequence (a decode step)
// takes a separate kernel that maps thread -> (row, vector) directly.
//
// Slot ownership: the first K-1 rows of a sequence (its "head", the rows that read
// history) are processed by the tile that holds the sequence's first row, even
// when they run past that tile's end; the next tile skips them.  That thread reads
// the slot (unless fresh) into registers and then writes the new state, so every
// slot element is read and written by one thread, in program order, and one
// launch serves any mix of run lengths (decode included).
#include "common.h"

namespace m2 {
namespace {

__device__ __forceinline__ int seq_of_row(const int32_t* __restrict__ cu, int S, int row) {
  // largest s in [0, S) with cu[s] <= row (cu is strictly increasing, cu[S] > row)
  int lo = 0, hi = S - 1;
  while (lo < hi) {
    int mid = (lo + hi + 1) >> 1;
    if (cu[mid] <= row)
      lo = mid;
    else
      hi = mid - 1;
  }
  return lo;
}

// 16 bytes of input read once by the launch: a non-temporal load, so the stream of rows
// does not displace cached data (the next kernels' inputs, pending writes).
template <typename T>
__device__ __forceinline__ uint4 load_stream(const T* p) {
  typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
  const u32x4 v = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
  return make_uint4(v.x, v.y, v.z, v.w);
}

template <typename T, int K>
__global__ __launch_bounds__(256) void conv1d_silu_kernel(
    T* __restrict__ dst, const T* __restrict__ x, const float* __restrict__ w,
    const float* __restrict__ b, T* __restrict__ conv_state, const int32_t* __restrict__ cu,
    const int32_t* __restrict__ slots, const uint8_t* __restrict__ fresh, int S, int T_rows,
    int Dc, int R, int64_t nthreads) {
  constexpr int V = Act<T>::kVec;
  constexpr int H1 = K - 1;
  const int64_t gid = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (gid >= nthreads) return;
  const int NV = Dc / V;
  const int v = (int)(gid % NV);
  const int tile = (int)(gid / NV);
  const int a = tile * R;
  const int bnd = min(T_rows, a + R);
  const size_t col = (size_t)v * V;

  // the thread's weights (V * K contiguous floats) and biases in 16-byte loads
  float wr[V][K], br[V];
  {
    const float4* wp = reinterpret_cast<const float4*>(w + col * K);
#pragma unroll
    for (int i = 0; i < V * K / 4; ++i) {
      const float4 t4 = wp[i];
      const float f[4] = {t4.x, t4.y, t4.z, t4.w};
#pragma unroll
      for (int e = 0; e < 4; ++e) wr[(4 * i + e) / K][(4 * i + e) % K] = f[e];
    }
    const float4* bp = reinterpret_cast<const float4*>(b + col);
#pragma unroll
    for (int i = 0; i < V / 4; ++i) {
      const float4 t4 = bp[i];
      br[4 * i] = t4.x;
      br[4 * i + 1] = t4.y;
      br[4 * i + 2] = t4.z;
      br[4 * i + 3] = t4.w;
    }
  }

  int s = seq_of_row(cu, S, a);
  int t = a;
  {
    const int st0 = cu[s], en = cu[s + 1];
    if (st0 < a) t = max(a, min(st0 + H1, en));  // head rows belong to an earlier tile
  }

  float win[H1][V];
  for (;;) {
    while (t >= cu[s + 1]) {
      if (++s >= S) return;
    }
    const int st0 = cu[s], en = cu[s + 1];
    if (st0 >= bnd) return;
    const bool own_head = st0 >= a;
    const int run_end = own_head ? min(en, max(bnd, st0 + H1)) : min(en, bnd);
    if (t >= run_end) return;

    if (t == st0) {
      // Sequence start (own_head): read the history, then write the new state.
      const size_t sbase = (size_t)slots[s] * H1 * Dc + col;
      uint4 raw[H1];
#pragma unroll
      for (int r = 0; r < H1; ++r) raw[r] = make_uint4(0, 0, 0, 0);
      if (!fresh[s]) {  // a fresh sequence never reads its slot
#pragma unroll
        for (int r = 0; r < H1; ++r)
          raw[r] = *reinterpret_cast<const uint4*>(conv_state + sbase + (size_t)r * Dc);
      }
#pragma unroll
      for (int r = 0; r < H1; ++r) Act<T>::unpack(raw[r], win[r]);
      const int L = en - st0;
      // new state row r = win[L + r]: history rows shifted up by L (constant indices
      // only, so raw stays in registers), then rows of the sequence
      uint4 nst[H1];
#pragma unroll
      for (int r = 0; r < H1; ++r) nst[r] = raw[r];
#pragma unroll
      for (int step = 0; step < H1; ++step) {
        if (step < L) {
#pragma unroll
          for (int r = 0; r + 1 < H1; ++r) nst[r] = nst[r + 1];
        }
      }
#pragma unroll
      for (int r = 0; r < H1; ++r) {
        const int idx = L + r;  // position in win = history ++ rows
        if (idx >= H1) nst[r] = *reinterpret_cast<const uint4*>(x + (size_t)(st0 + idx - H1) * Dc + col);
      }
#pragma unroll
      for (int r = 0; r < H1; ++r)
        *reinterpret_cast<uint4*>(conv_state + sbase + (size_t)r * Dc) = nst[r];
    } else {
      // Mid-sequence entry: t >= st0 + H1, the window comes from the rows before t.
#pragma unroll
      for (int r = 0; r < H1; ++r)
        Act<T>::unpack(*reinterpret_cast<const uint4*>(x + (size_t)(t - H1 + r) * Dc + col), win[r]);
    }

    while (t < run_end) {
      // four rows at a time: the window holds the K-1 previous rows, then the four new ones
      const int n = min(4, run_end - t);
      float xf[H1 + 4][V];
#pragma unroll
      for (int r = 0; r < H1; ++r)
#pragma unroll
        for (int i = 0; i < V; ++i) xf[r][i] = win[r][i];
      uint4 xv[4];
#pragma unroll
      for (int j = 0; j < 4; ++j)
        xv[j] = j < n ? load_stream(x + (size_t)(t + j) * Dc + col) : make_uint4(0, 0, 0, 0);
#pragma unroll
      for (int j = 0; j < 4; ++j) Act<T>::unpack(xv[j], xf[H1 + j]);
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        if (j < n) {
          float out[V];
#pragma unroll
          for (int i = 0; i < V; ++i) {
            float pre = br[i];
#pragma unroll
            for (int k = 0; k < K; ++k) pre = fmaf(wr[i][k], xf[j + k][i], pre);
            out[i] = silu_f32(pre);
          }
          *reinterpret_cast<uint4*>(dst + (size_t)(t + j) * Dc + col) = Act<T>::pack(out);
        }
      }
      // the window for the next rows: the last K-1 of the K-1 + n rows
#pragma unroll
      for (int r = 0; r < H1; ++r)
#pragma unroll
        for (int i = 0; i < V; ++i) {
          float v = xf[r + 4][i];
          if (n < 4) v = n == 3 ? xf[r + 3][i] : (n == 2 ? xf[r + 2][i] : xf[r + 1][i]);
          win[r][i] = v;
        }
      t += n;
    }
    if (t >= bnd) return;
  }
}

// Every sequence one row (a decode step: S == T, so row r is sequence r): one thread per
// 16-byte channel vector of a row, one wave per 64 vectors of a row (grid x), rows over grid y
// (strided past the grid's y limit), so the row's slot index and fresh flag are uniform
// scalar loads and no lane divides by the row width.  The slot's K-1 rows and the new row
// are read together, the output is the window's dot product, and the slot is rewritten
// shifted by one row.  The only dependent load is the slot's rows, after the slot index.
template <typename T, int K>
__global__ __launch_bounds__(64) void conv1d_silu_step_kernel(
    T* __restrict__ dst, const T* __restrict__ x, const float* __restrict__ w,
    const float* __restrict__ b, T* __restrict__ conv_state, const int32_t* __restrict__ slots,
    const uint8_t* __restrict__ fresh, int S, int Dc) {
  constexpr int V = Act<T>::kVec;
  constexpr int H1 = K - 1;
  const int NV = Dc / V;
  const int vec = blockIdx.x * 64 + threadIdx.x;
  if (vec >= NV) return;
  const size_t col = (size_t)vec * V;
  // weights of this thread's channels: V * K contiguous floats starting at col * K
  float wr[V * K];
  const float4* wp = reinterpret_cast<const float4*>(w + col * K);
#pragma unroll
  for (int i = 0; i < V * K / 4; ++i) {
    const float4 t4 = wp[i];
    wr[4 * i] = t4.x;
    wr[4 * i + 1] = t4.y;
    wr[4 * i + 2] = t4.z;
    wr[4 * i + 3] = t4.w;
  }
  float br[V];
  const float4* bp = reinterpret_cast<const float4*>(b + col);
#pragma unroll
  for (int i = 0; i < V / 4; ++i) {
    const float4 t4 = bp[i];
    br[4 * i] = t4.x;
    br[4 * i + 1] = t4.y;
    br[4 * i + 2] = t4.z;
    br[4 * i + 3] = t4.w;
  }
  for (int r = blockIdx.y; r < S; r += gridDim.y) {
    uint4 raw[K];
    raw[H1] = *reinterpret_cast<const uint4*>(x + (size_t)r * Dc + col);
    const size_t sbase = (size_t)slots[r] * H1 * Dc + col;
#pragma unroll
    for (int i = 0; i < H1; ++i) raw[i] = make_uint4(0, 0, 0, 0);
    if (!fresh[r]) {  // a fresh sequence never reads its slot
#pragma unroll
      for (int i = 0; i < H1; ++i) raw[i] = *reinterpret_cast<const uint4*>(conv_state + sbase + (size_t)i * Dc);
    }
#pragma unroll
    for (int i = 0; i < H1; ++i) *reinterpret_cast<uint4*>(conv_state + sbase + (size_t)i * Dc) = raw[i + 1];
    float win[K][V];
#pragma unroll
    for (int k = 0; k < K; ++k) Act<T>::unpack(raw[k], win[k]);
    float out[V];
#pragma unroll
    for (int i = 0; i < V; ++i) {
      float pre = br[i];
#pragma unroll
      for (int k = 0; k < K; ++k) pre = fmaf(wr[i * K + k], win[k][i], pre);
      out[i] = silu_f32(pre);
    }
    *reinterpret_cast<uint4*>(dst + (size_t)r * Dc + col) = Act<T>::pack(out);
  }
}

template <typename T, int K>
hipError_t launch_t(void* dst, const void* x, const float* w, const float* b, void* cs,
                    const BatchDev& bd, int32_t Dc, hipStream_t st) {
  constexpr int V = Act<T>::kVec;
  const int NV = Dc / V;
  if (bd.num_rows == bd.num_seqs) {
    const dim3 grid((unsigned)((NV + 63) / 64), (unsigned)(bd.num_seqs < 65535 ? bd.num_seqs : 65535));
    M2_LAUNCH("conv1d_silu", (conv1d_silu_step_kernel<T, K>), grid, dim3(64), 0, st, (T*)dst, (const T*)x, w, b,
              (T*)cs, bd.slots, bd.fresh, bd.num_seqs, Dc);
    return hipSuccess;
  }
  const int64_t work = (int64_t)bd.num_rows * NV;
  // rows per thread: enough threads to fill the chip (~512K), 4 to 32 rows each (fewer than
  // 4 would reload each thread's weights for too little work: 19 us -> 9 us on 2048 rows)
  int R = (int)((work + 524287) / 524288);
  R = R < 4 ? 4 : (R > 32 ? 32 : R);
  const int64_t tiles = (bd.num_rows + R - 1) / R;
  const int64_t nthreads = tiles * NV;
  const dim3 grid((unsigned)((nthreads + 255) / 256));
  M2_LAUNCH("conv1d_silu", (conv1d_silu_kernel<T, K>), grid, dim3(256), 0, st, (T*)dst,
            (const T*)x, w, b, (T*)cs, bd.cu_seqlens, bd.slots, bd.fresh, bd.num_seqs, bd.num_rows,
            Dc, R, nthreads);
  return hipSuccess;
}

}  // namespace

hipError_t launch_conv1d(void* dst, const void* x, const float* w, const float* b, void* cs,
                         const BatchDev& bd, int32_t Dc, int32_t K, int32_t act, hipStream_t st) {
  if (act == MAMBA2_DTYPE_BF16) {
    switch (K) {
      case 2: return launch_t<bf16_t, 2>(dst, x, w, b, cs, bd, Dc, st);
      case 3: return launch_t<bf16_t, 3>(dst, x, w, b, cs, bd, Dc, st);
      case 4: return launch_t<bf16_t, 4>(dst, x, w, b, cs, bd, Dc, st);
    }
  } else {
    switch (K) {
      case 2: return launch_t<float, 2>(dst, x, w, b, cs, bd, Dc, st);
      case 3: return launch_t<float, 3>(dst, x, w, b, cs, bd, Dc, st);
      case 4: return launch_t<float, 4>(dst, x, w, b, cs, bd, Dc, st);
    }
  }
  return hipErrorInvalidValue;
}

}  // namespace m2
