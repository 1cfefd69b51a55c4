// Chunked selective scan on MFMA for gfx950: bf16 activations, headdim 64, d_state 128.
//
// The recurrence ("feat(backend): Mamba2 ops, with CPU reference implementations",
// section "Ops", SSMScan) summed in closed form over chunks of 64 rows ("Granite Mamba2
// Inference Optimization": long prefill as a chunked parallel scan).  Per chunk, with
// a_t = -exp(A_log) dt'_t and cs_i = sum_{t<=i} a_t inside the chunk, for every head:
//   y_i   = sum_{j<=i} (C_i . B_j) exp(cs_i - cs_j) dt'_j x_j + exp(cs_i) C_i . S + D x_i
//   S'    = exp(cs_63) S + sum_j exp(cs_63 - cs_j) dt'_j x_j (x) B_j
// with S the state entering the chunk.  The contractions run on v_mfma_f32_16x16x32_bf16
// (fp32 accumulate):
//   G^T = B C^T        (64 x 64, K = N = 128), once per chunk, shared by the heads of the
//                      workgroup (one B/C group)
//   Y^T = S C^T (scaled by exp(cs_i)) + X^T M^T   with M = G o decay mask o dt' taken
//                      straight from the G^T accumulators (their lane layout is the MFMA
//                      B-operand layout, the K index permuted consistently on both
//                      operands)
//   S^T = exp(cs_63) S^T + B^T (w o X),  w_j = exp(cs_63 - cs_j) dt'_j.
// x, B and C are exact in bf16.  M, S and w o X are fp32 values split into bf16 hi + lo
// halves (two MFMAs each): y sums terms that cancel, so one bf16 rounding of M or of a
// large, slowly decaying S moves outputs past the bf16 output bar, and the fp32 state
// needs ~16 bits per step.
//
// Workgroup: 4 waves, 2 heads, one segment (a run of chunks of one sequence).  Wave w owns
// output rows 16w..16w+15 of the chunk and state rows n in [32w, 32w+32).  The state stays
// in MFMA accumulator registers across the segment's chunks.  LDS (~74 KiB, so two
// workgroups share a CU) holds the chunk's B rows, the head's X^T, (w o X)^T hi/lo and
// S hi/lo; tiles are XOR-swizzled in 16-byte units so that the 16 lanes reading 16
// different rows of one column block hit distinct banks.
#include "common.h"

namespace m2 {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr int kP = 64;   // head dim
constexpr int kN = 128;  // state dim
constexpr int kQ = 64;   // chunk rows
constexpr int kHB = 2;   // heads per workgroup

// Swizzled element offsets (16-byte units of 8 bf16 are XOR-permuted per row).
__device__ __forceinline__ int off_pj(int p, int j) {  // [64][64] tiles indexed [p][j]
  return p * kQ + ((((j >> 3) ^ (p >> 1)) & 7) << 3) + (j & 7);
}
__device__ __forceinline__ int off_pn(int p, int n) {  // [64][128] S tiles [p][n]
  return p * kN + ((((n >> 3) ^ p) & 15) << 3) + (n & 7);
}
__device__ __forceinline__ int off_jn(int j, int n) {  // [64][128] B rows [j][n]
  return j * kN + ((((n >> 3) ^ j) & 15) << 3) + (n & 7);
}

struct Decay {
  float cs[kHB][kQ];   // cs_i
  float dtp[kHB][kQ];  // dt'_j
  float W[kHB][kQ];    // exp(cs_63 - cs_j) dt'_j, from suffix sums
  float dch[kHB];      // exp(cs_63)
  float lsum[kHB];     // sum of a over the segment so far
};

struct Smem {
  bf16_t B[kQ * kN];     // B rows [j][n]
  bf16_t XT[kP * kQ];    // X^T [p][j]
  bf16_t WXh[kP * kQ];   // (w o X)^T hi [p][j]
  bf16_t WXl[kP * kQ];   // (w o X)^T lo
  bf16_t Sh[kP * kN];    // S hi [p][n]
  bf16_t Sl[kP * kN];    // S lo
  Decay d;
};

struct SmemState {
  bf16_t B[kQ * kN];
  bf16_t WXh[kP * kQ];
  bf16_t WXl[kP * kQ];
  Decay d;
};

__device__ __forceinline__ f32x4 mfma(const bf16x8& a, const bf16x8& b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ uint32_t pk(float lo, float hi) {
  bf16x2 v = {(__bf16)lo, (__bf16)hi};
  return __builtin_bit_cast(uint32_t, v);
}

__device__ __forceinline__ float lo_f(uint32_t u) { return __uint_as_float(u << 16); }
__device__ __forceinline__ float hi_f(uint32_t u) { return __uint_as_float(u & 0xffff0000u); }
__device__ __forceinline__ float bf_round(float v) { return (float)(__bf16)v; }

__device__ __forceinline__ bf16x8 as_bf8(const u32x4& v) { return __builtin_bit_cast(bf16x8, v); }

template <typename T>
__device__ __forceinline__ u32x4 ld16(const T* p) { return *reinterpret_cast<const u32x4*>(p); }
template <typename T>
__device__ __forceinline__ u32x2 ld8(const T* p) { return *reinterpret_cast<const u32x2*>(p); }
template <typename T>
__device__ __forceinline__ void st8(T* p, u32x2 v) { *reinterpret_cast<u32x2*>(p) = v; }
template <typename T>
__device__ __forceinline__ void st16(T* p, u32x4 v) { *reinterpret_cast<u32x4*>(p) = v; }

__device__ __forceinline__ float wave_scan_incl(float v, int lane) {
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const float t = __shfl_up(v, o, 64);
    if (lane >= o) v += t;
  }
  return v;
}

__device__ __forceinline__ float wave_rscan_incl(float v, int lane) {
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const float t = __shfl_down(v, o, 64);
    if (lane + o < 64) v += t;
  }
  return v;
}

struct SegPtrs {
  const int2* seq_info;
  const int4* seg_info;
  float* seg_decay;
  float* seg_state;
};

// The chunk's B rows (64 x 128 bf16) into LDS, zero past the segment's last row.
__device__ __forceinline__ void fill_b(bf16_t* sB, const bf16_t* __restrict__ xbc, size_t Dc, size_t boff,
                                       int r0, int nr) {
  const int t = threadIdx.x;
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    const int u = t + 256 * k;  // 16-byte unit: row u / 16, columns 8 (u % 16)
    const int j = u >> 4, n = (u & 15) * 8;
    const u32x4 v = j < nr ? ld16(xbc + (size_t)(r0 + j) * Dc + boff + n) : u32x4{0, 0, 0, 0};
    st16(sB + off_jn(j, n), v);
  }
}

// X^T (optional) and (w o X)^T hi/lo of one head: thread t transposes 4 rows x 4 columns.
template <bool kWithX, typename SM>
__device__ __forceinline__ void fill_x(SM& sm, const bf16_t* __restrict__ xbc, size_t Dc, size_t xoff, int r0,
                                       int nr, int hh) {
  const int t = threadIdx.x;
  const int jq = t >> 4;  // rows 4jq..4jq+3
  const int pq = t & 15;  // columns 4pq..4pq+3
  u32x2 v[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int j = 4 * jq + i;
    v[i] = j < nr ? ld8(xbc + (size_t)(r0 + j) * Dc + xoff + 4 * pq) : u32x2{0, 0};
  }
  const f32x4 w = *reinterpret_cast<const f32x4*>(&sm.d.W[hh][4 * jq]);
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    const int p = 4 * pq + e;
    float xf[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const uint32_t dd = v[i][e >> 1];
      xf[i] = (e & 1) ? hi_f(dd) : lo_f(dd);
    }
    if constexpr (kWithX) st8(&sm.XT[off_pj(p, 4 * jq)], u32x2{pk(xf[0], xf[1]), pk(xf[2], xf[3])});
    float hi[4], lo[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const float wx = w[i] * xf[i];
      hi[i] = bf_round(wx);
      lo[i] = wx - hi[i];
    }
    st8(&sm.WXh[off_pj(p, 4 * jq)], u32x2{pk(hi[0], hi[1]), pk(hi[2], hi[3])});
    st8(&sm.WXl[off_pj(p, 4 * jq)], u32x2{pk(lo[0], lo[1]), pk(lo[2], lo[3])});
  }
}

// dt' and the decay sums of one head for the chunk (one wave: lane = row).
__device__ __forceinline__ void chunk_decay(Decay& d, const bf16_t* __restrict__ dt, int H, int h, float A,
                                            float bias, int r0, int nr, int hh, int lane) {
  float dtp = 0.f;
  if (lane < nr) dtp = softplus_f32(bf16_to_f32(dt[(size_t)(r0 + lane) * H + h]) + bias);
  const float a = -A * dtp;
  const float cs = wave_scan_incl(a, lane);
  const float rs = wave_rscan_incl(a, lane);  // sum_{t >= lane} a_t
  float suf = __shfl_down(rs, 1, 64);         // sum_{t > lane} a_t
  if (lane == 63) suf = 0.f;
  d.cs[hh][lane] = cs;
  d.dtp[hh][lane] = dtp;
  d.W[hh][lane] = __expf(suf) * dtp;
  if (lane == 63) {
    d.dch[hh] = __expf(cs);
    d.lsum[hh] += cs;
  }
}

// B^T operands of wave w: rows n = 32w + 16nb + c, k = j = 32m + 8g + s (from LDS B rows).
__device__ __forceinline__ void load_bt_ops(const bf16_t* sB, u32x4 (&bt)[2][2], int w, int lane) {
  const int g = lane >> 4, c = lane & 15;
#pragma unroll
  for (int nb = 0; nb < 2; ++nb) {
    const int n = 32 * w + 16 * nb + c;
#pragma unroll
    for (int m = 0; m < 2; ++m) {
      uint32_t e[8];
#pragma unroll
      for (int k = 0; k < 8; ++k) e[k] = sB[off_jn(32 * m + 8 * g + k, n)];
      bt[nb][m] = u32x4{e[0] | (e[1] << 16), e[2] | (e[3] << 16), e[4] | (e[5] << 16), e[6] | (e[7] << 16)};
    }
  }
}

// S^T (8 tiles of wave w) <- dch S^T + B^T (w o X), the operand in hi and lo halves.
template <typename SM>
__device__ __forceinline__ void state_update(const SM& sm, f32x4 (&S)[8], int hh, int w, int lane) {
  const int g = lane >> 4, c = lane & 15;
  u32x4 bt[2][2];
  load_bt_ops(sm.B, bt, w, lane);
  const float d = sm.d.dch[hh];
#pragma unroll
  for (int t = 0; t < 8; ++t) S[t] *= d;
#pragma unroll
  for (int pb = 0; pb < 4; ++pb) {
    const int p = 16 * pb + c;
#pragma unroll
    for (int m = 0; m < 2; ++m) {
      const int off = off_pj(p, 32 * m + 8 * g);
      const bf16x8 bh = as_bf8(ld16(&sm.WXh[off]));
      const bf16x8 bl = as_bf8(ld16(&sm.WXl[off]));
#pragma unroll
      for (int nb = 0; nb < 2; ++nb) {
        const bf16x8 a = as_bf8(bt[nb][m]);
        S[4 * nb + pb] = mfma(a, bh, S[4 * nb + pb]);
        S[4 * nb + pb] = mfma(a, bl, S[4 * nb + pb]);
      }
    }
    __builtin_amdgcn_sched_barrier(0);
  }
}

// State tile t of wave w holds S[p][n..n+3], p = 16 (t % 4) + c, n = 32w + 16 (t / 4) + 4g.
__device__ __forceinline__ size_t state_elem(int t, int w, int lane) {
  const int g = lane >> 4, c = lane & 15;
  return (size_t)(16 * (t & 3) + c) * kN + 32 * w + 16 * (t >> 2) + 4 * g;
}

// ---------------------------------------------------------------- segment states

__global__ __launch_bounds__(256, 2) void ssd_mfma_state_kernel(const bf16_t* __restrict__ xbc,
                                                                const bf16_t* __restrict__ dt,
                                                                const float* __restrict__ a_log,
                                                                const float* __restrict__ dt_bias,
                                                                SegPtrs sp, int H, int G, int nhb) {
  __shared__ SmemState sm;
  const int seg = blockIdx.x / nhb;
  const int h0 = (blockIdx.x % nhb) * kHB;
  const int4 si = sp.seg_info[seg];
  const int2 qi = sp.seq_info[si.x];
  if (si.w == qi.y - 1) return;  // a sequence's last segment needs no local state
  const int tid = threadIdx.x, w = tid >> 6, lane = tid & 63;
  const int Di = H * kP;
  const size_t Dc = (size_t)Di + 2 * (size_t)G * kN;
  const size_t boff = (size_t)Di + (size_t)(h0 / (H / G)) * kN;
  if (tid < kHB) sm.d.lsum[tid] = 0.f;

  f32x4 S[kHB][8];
#pragma unroll
  for (int hh = 0; hh < kHB; ++hh)
#pragma unroll
    for (int t = 0; t < 8; ++t) S[hh][t] = f32x4{0.f, 0.f, 0.f, 0.f};

  const int nchunks = (si.z + kQ - 1) / kQ;
  for (int q = 0; q < nchunks; ++q) {
    const int r0 = si.y + q * kQ;
    const int nr = min(kQ, si.z - q * kQ);
    __syncthreads();  // the previous chunk is done with LDS
    fill_b(sm.B, xbc, Dc, boff, r0, nr);
    if (w < kHB) chunk_decay(sm.d, dt, H, h0 + w, __expf(a_log[h0 + w]), dt_bias[h0 + w], r0, nr, w, lane);
    __syncthreads();
#pragma unroll
    for (int hh = 0; hh < kHB; ++hh) {
      if (hh > 0) __syncthreads();  // the previous head is done with WX
      fill_x<false>(sm, xbc, Dc, (size_t)(h0 + hh) * kP, r0, nr, hh);
      __syncthreads();
      state_update(sm, S[hh], hh, w, lane);
    }
  }
#pragma unroll
  for (int hh = 0; hh < kHB; ++hh) {
    float* out = sp.seg_state + ((size_t)seg * H + h0 + hh) * (size_t)(kP * kN);
#pragma unroll
    for (int t = 0; t < 8; ++t) *reinterpret_cast<f32x4*>(out + state_elem(t, w, lane)) = S[hh][t];
  }
  if (tid < kHB) sp.seg_decay[(size_t)seg * H + h0 + tid] = __expf(sm.d.lsum[tid]);
}

// ---------------------------------------------------------------- outputs

__global__ __launch_bounds__(256, 2) void ssd_mfma_scan_kernel(
    bf16_t* __restrict__ y, const bf16_t* __restrict__ xbc, const bf16_t* __restrict__ dt,
    const float* __restrict__ a_log, const float* __restrict__ dt_bias, const float* __restrict__ Dp,
    float* __restrict__ pool, const int32_t* __restrict__ slots, SegPtrs sp, int H, int G, int nhb) {
  __shared__ Smem sm;
  const int seg = blockIdx.x / nhb;
  const int h0 = (blockIdx.x % nhb) * kHB;
  const int4 si = sp.seg_info[seg];
  const int2 qi = sp.seq_info[si.x];
  const bool last = si.w == qi.y - 1;
  const int tid = threadIdx.x, w = tid >> 6, lane = tid & 63;
  const int g = lane >> 4, c = lane & 15;
  const int Di = H * kP;
  const size_t Dc = (size_t)Di + 2 * (size_t)G * kN;
  const int grp = h0 / (H / G);
  const size_t boff = (size_t)Di + (size_t)grp * kN;
  const size_t coff = (size_t)Di + (size_t)G * kN + (size_t)grp * kN;
  const int irow = 16 * w + c;  // this lane's output row in the chunk
  if (tid < kHB) sm.d.lsum[tid] = 0.f;

  // the state entering the segment (written by the pass kernel)
  f32x4 S[kHB][8];
#pragma unroll
  for (int hh = 0; hh < kHB; ++hh) {
    const float* in = sp.seg_state + ((size_t)seg * H + h0 + hh) * (size_t)(kP * kN);
#pragma unroll
    for (int t = 0; t < 8; ++t) S[hh][t] = *reinterpret_cast<const f32x4*>(in + state_elem(t, w, lane));
  }

  const int nchunks = (si.z + kQ - 1) / kQ;
  for (int q = 0; q < nchunks; ++q) {
    const int r0 = si.y + q * kQ;
    const int nr = min(kQ, si.z - q * kQ);
    __syncthreads();  // the previous chunk is done with LDS
    fill_b(sm.B, xbc, Dc, boff, r0, nr);
    if (w < kHB) chunk_decay(sm.d, dt, H, h0 + w, __expf(a_log[h0 + w]), dt_bias[h0 + w], r0, nr, w, lane);
    // C rows of this wave's row block: the B-operand of G^T and of S C^T (k = n, col = i)
    u32x4 cr[4];
#pragma unroll
    for (int kk = 0; kk < 4; ++kk)
      cr[kk] = irow < nr ? ld16(xbc + (size_t)(r0 + irow) * Dc + coff + 32 * kk + 8 * g) : u32x4{0, 0, 0, 0};
    __syncthreads();
    // G^T tiles (j block jb, i block w), jb <= w
    f32x4 Gt[4];
#pragma unroll
    for (int jb = 0; jb < 4; ++jb) {
      Gt[jb] = f32x4{0.f, 0.f, 0.f, 0.f};
      if (jb <= w) {
#pragma unroll
        for (int kk = 0; kk < 4; ++kk)
          Gt[jb] = mfma(as_bf8(ld16(&sm.B[off_jn(16 * jb + c, 32 * kk + 8 * g)])), as_bf8(cr[kk]), Gt[jb]);
      }
    }

#pragma unroll
    for (int hh = 0; hh < kHB; ++hh) {
      const int h = h0 + hh;
      if (hh > 0) __syncthreads();  // the previous head is done with XT, WX and S
      fill_x<true>(sm, xbc, Dc, (size_t)h * kP, r0, nr, hh);
      // S [p][n] in bf16 hi + lo halves
#pragma unroll
      for (int t = 0; t < 8; ++t) {
        const int p = 16 * (t & 3) + c;
        const int n = 32 * w + 16 * (t >> 2) + 4 * g;
        float lo[4];
#pragma unroll
        for (int r = 0; r < 4; ++r) lo[r] = S[hh][t][r] - bf_round(S[hh][t][r]);
        st8(&sm.Sh[off_pn(p, n)], u32x2{pk(S[hh][t][0], S[hh][t][1]), pk(S[hh][t][2], S[hh][t][3])});
        st8(&sm.Sl[off_pn(p, n)], u32x2{pk(lo[0], lo[1]), pk(lo[2], lo[3])});
      }
      __syncthreads();

      // ---- Y^T tiles (p block pb, i block w): exp(cs_i) S C^T + X^T M^T + D x ----
      const float csi = sm.d.cs[hh][irow];
      const float ei = __expf(csi);
      f32x4 yacc[4];
#pragma unroll
      for (int pb = 0; pb < 4; ++pb) {
        yacc[pb] = f32x4{0.f, 0.f, 0.f, 0.f};
        const int p = 16 * pb + c;
#pragma unroll
        for (int kk = 0; kk < 4; ++kk) {
          const int off = off_pn(p, 32 * kk + 8 * g);
          yacc[pb] = mfma(as_bf8(ld16(&sm.Sh[off])), as_bf8(cr[kk]), yacc[pb]);
          yacc[pb] = mfma(as_bf8(ld16(&sm.Sl[off])), as_bf8(cr[kk]), yacc[pb]);
        }
        yacc[pb] *= ei;
        __builtin_amdgcn_sched_barrier(0);
      }
      // M^T operands, hi and lo: slots 0..3 from G^T tile 2m, slots 4..7 from tile 2m + 1
#pragma unroll
      for (int m = 0; m < 2; ++m) {
        if (m <= (w >> 1)) {
          float mv[8];
#pragma unroll
          for (int half = 0; half < 2; ++half) {
            const int jb = 2 * m + half;
            const int j0 = 16 * jb + 4 * g;
            const f32x4 csj = *reinterpret_cast<const f32x4*>(&sm.d.cs[hh][j0]);
            const f32x4 dtj = *reinterpret_cast<const f32x4*>(&sm.d.dtp[hh][j0]);
#pragma unroll
            for (int r = 0; r < 4; ++r) {
              float v = 0.f;
              if (jb <= w && j0 + r <= irow) v = Gt[jb][r] * __expf(csi - csj[r]) * dtj[r];
              mv[4 * half + r] = v;
            }
          }
          u32x4 mh, ml;
#pragma unroll
          for (int k = 0; k < 4; ++k) {
            mh[k] = pk(mv[2 * k], mv[2 * k + 1]);
            ml[k] = pk(mv[2 * k] - bf_round(mv[2 * k]), mv[2 * k + 1] - bf_round(mv[2 * k + 1]));
          }
#pragma unroll
          for (int pb = 0; pb < 4; ++pb) {
            const int p = 16 * pb + c;
            const u32x2 x0 = ld8(&sm.XT[off_pj(p, 32 * m + 4 * g)]);
            const u32x2 x1 = ld8(&sm.XT[off_pj(p, 32 * m + 16 + 4 * g)]);
            const bf16x8 xo = as_bf8(u32x4{x0.x, x0.y, x1.x, x1.y});
            yacc[pb] = mfma(xo, as_bf8(mh), yacc[pb]);
            yacc[pb] = mfma(xo, as_bf8(ml), yacc[pb]);
          }
          __builtin_amdgcn_sched_barrier(0);
        }
      }
      // + D x and store: lane holds y[i = irow][p = 16pb + 4g + r]
      if (irow < nr) {
        const float dh = Dp[h];
        const size_t rowoff = (size_t)(r0 + irow) * Dc + (size_t)h * kP;
        bf16_t* yrow = y + (size_t)(r0 + irow) * Di + (size_t)h * kP;
#pragma unroll
        for (int pb = 0; pb < 4; ++pb) {
          const int p0 = 16 * pb + 4 * g;
          const u32x2 xv = ld8(xbc + rowoff + p0);
          st8(yrow + p0, u32x2{pk(fmaf(dh, lo_f(xv.x), yacc[pb][0]), fmaf(dh, hi_f(xv.x), yacc[pb][1])),
                               pk(fmaf(dh, lo_f(xv.y), yacc[pb][2]), fmaf(dh, hi_f(xv.y), yacc[pb][3]))});
        }
      }
      // ---- state update ----
      __builtin_amdgcn_sched_barrier(0);
      state_update(sm, S[hh], hh, w, lane);
      __builtin_amdgcn_sched_barrier(0);
    }
  }
  if (last) {
    const int s = si.x;
#pragma unroll
    for (int hh = 0; hh < kHB; ++hh) {
      float* out = pool + ((size_t)slots[s] * H + h0 + hh) * (size_t)(kP * kN);
#pragma unroll
      for (int t = 0; t < 8; ++t) *reinterpret_cast<f32x4*>(out + state_elem(t, w, lane)) = S[hh][t];
    }
  }
}

}  // namespace

// Shapes the MFMA path covers: bf16, P = 64, N = 128, heads in pairs within one group.
bool scan_mfma_supported(const mamba2_dims* d) {
  return d->act_dtype == MAMBA2_DTYPE_BF16 && d->headdim == kP && d->d_state == kN && d->nheads % kHB == 0 &&
         (d->nheads / d->ngroups) % kHB == 0;
}

hipError_t launch_scan_mfma(const ScanArgs& a, hipStream_t st) {
  const SegPtrs sp{(const int2*)(a.ws + a.lay.off_seq_info), (const int4*)(a.ws + a.lay.off_seg_info),
                   (float*)(a.ws + a.lay.off_seg_decay), (float*)(a.ws + a.lay.off_seg_state)};
  const mamba2_dims& d = a.dims;
  const int nhb = d.nheads / kHB;
  const dim3 grid((unsigned)(a.lay.nseg * nhb));
  M2_LAUNCH("ssd_state", ssd_mfma_state_kernel, grid, dim3(256), 0, st, (const bf16_t*)a.xbc,
            (const bf16_t*)a.dt, a.a_log, a.dt_bias, sp, d.nheads, d.ngroups, nhb);
  hipError_t e = launch_scan_pass(a, st);
  if (e != hipSuccess) return e;
  M2_LAUNCH("ssd_scan", ssd_mfma_scan_kernel, grid, dim3(256), 0, st, (bf16_t*)a.y, (const bf16_t*)a.xbc,
            (const bf16_t*)a.dt, a.a_log, a.dt_bias, a.D, a.ssm_state, a.bd.slots, sp, d.nheads, d.ngroups,
            nhb);
  return hipSuccess;
}

}  // namespace m2
