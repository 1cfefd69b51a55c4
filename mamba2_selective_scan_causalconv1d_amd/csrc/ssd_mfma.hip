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
//   G^T = B C^T        (64 x 64, K = N = 128)
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
// Two kernels walk a segment (a run of chunks of one sequence) per workgroup of 4 waves:
//   ssd_state: the segment's local end state (from zero), two heads per workgroup;
//   ssd_scan:  y for one head from the state entering the segment (which the pass kernel
//              supplies), and the final state for a sequence's last segment.
// Wave w owns output rows 16w..16w+15 of a chunk and state rows n in [32w, 32w+32); the
// state stays in MFMA accumulator registers across the segment.  The global loads of chunk
// q+1 (B rows, x, C rows, dt) are issued into registers while chunk q computes.  LDS tiles
// are XOR-swizzled in 16-byte units so that 16 lanes reading 16 rows of one column block
// hit distinct banks; chunk rows are read and written through buffer resources (a
// wave-uniform base and 32-bit lane offsets).
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

// Swizzled element offsets (16-byte units of 8 bf16 XOR-permuted per row).
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
  float cs[kQ];   // cs_i
  float dtp[kQ];  // dt'_j
  float W[kQ];    // exp(cs_63 - cs_j) dt'_j, from suffix sums
  float dch;      // exp(cs_63)
  float lsum;     // sum of a over the segment so far
  float pad[2];
};

struct SmemScan {
  bf16_t B[kQ * kN];    // B rows [j][n]
  bf16_t XT[kP * kQ];   // X^T [p][j]
  bf16_t WXh[kP * kQ];  // (w o X)^T hi [p][j]
  bf16_t WXl[kP * kQ];  // (w o X)^T lo
  bf16_t Sh[kP * kN];   // S hi [p][n]
  bf16_t Sl[kP * kN];   // S lo
  Decay d;
};

struct SmemState {
  bf16_t B[kQ * kN];
  bf16_t WXh[2][kP * kQ];
  bf16_t WXl[2][kP * kQ];
  Decay d[2];
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

// Buffer resources over the rows of one chunk: a wave-uniform base and a byte range, so
// every access is a 32-bit lane offset, and offsets at or past the range (the rows after
// the segment's last row) read as zero and drop writes.
typedef __amdgpu_buffer_rsrc_t Rsrc;
__device__ __forceinline__ Rsrc rows_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, (int)bytes, 0x00020000);
}
__device__ __forceinline__ u32x4 bld16(Rsrc r, uint32_t off) {
  return __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 0);
}
__device__ __forceinline__ u32x2 bld8(Rsrc r, uint32_t off) {
  return __builtin_amdgcn_raw_buffer_load_b64(r, off, 0, 0);
}
__device__ __forceinline__ void bst8(Rsrc r, uint32_t off, u32x2 v) {
  __builtin_amdgcn_raw_buffer_store_b64(v, r, off, 0, 0);
}
__device__ __forceinline__ int uniform(int v) { return __builtin_amdgcn_readfirstlane(v); }

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

// ------------------------------------------------------------ per-chunk loads (registers)

// B rows of a chunk: thread t holds 16-byte units u = t + 256k (row u / 16, columns 8 (u % 16)).
struct PfB {
  u32x4 v[4];
};
__device__ __forceinline__ void load_b(PfB& p, Rsrc rows, uint32_t ld, uint32_t col) {
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    const uint32_t u = threadIdx.x + 256u * k;
    p.v[k] = bld16(rows, 2u * ((u >> 4) * ld + col + (u & 15u) * 8u));
  }
}
__device__ __forceinline__ void store_b(bf16_t* sB, const PfB& p) {
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    const int u = (int)threadIdx.x + 256 * k;
    st16(sB + off_jn(u >> 4, (u & 15) * 8), p.v[k]);
  }
}

// x of one head: thread t holds rows 4jq..4jq+3 (jq = t / 16), columns 4pq..4pq+3 (pq = t % 16).
struct PfX {
  u32x2 v[4];
};
__device__ __forceinline__ void load_x(PfX& p, Rsrc rows, uint32_t ld, uint32_t col) {
  const uint32_t jq = threadIdx.x >> 4, pq = threadIdx.x & 15;
#pragma unroll
  for (int i = 0; i < 4; ++i) p.v[i] = bld8(rows, 2u * ((4u * jq + i) * ld + col + 4u * pq));
}

// X^T (optional) and (w o X)^T hi/lo from the registers: a 4 x 4 transpose per thread.
template <bool kWithX>
__device__ __forceinline__ void store_x(bf16_t* XT, bf16_t* WXh, bf16_t* WXl, const PfX& px, const float* W) {
  const int jq = threadIdx.x >> 4, pq = threadIdx.x & 15;
  const f32x4 w = *reinterpret_cast<const f32x4*>(&W[4 * jq]);
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    const int p = 4 * pq + e;
    float xf[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const uint32_t dd = px.v[i][e >> 1];
      xf[i] = (e & 1) ? hi_f(dd) : lo_f(dd);
    }
    if constexpr (kWithX) st8(&XT[off_pj(p, 4 * jq)], u32x2{pk(xf[0], xf[1]), pk(xf[2], xf[3])});
    float hi[4], lo[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const float wx = w[i] * xf[i];
      hi[i] = bf_round(wx);
      lo[i] = wx - hi[i];
    }
    st8(&WXh[off_pj(p, 4 * jq)], u32x2{pk(hi[0], hi[1]), pk(hi[2], hi[3])});
    st8(&WXl[off_pj(p, 4 * jq)], u32x2{pk(lo[0], lo[1]), pk(lo[2], lo[3])});
  }
}

// dt' and the decay sums of one head for the chunk (one wave: lane = row; v = dt, raw).
__device__ __forceinline__ void chunk_decay(Decay& d, float v, float A, float bias, int nr, int lane) {
  const float dtp = lane < nr ? softplus_f32(v + bias) : 0.f;
  const float a = -A * dtp;
  const float cs = wave_scan_incl(a, lane);
  const float rs = wave_rscan_incl(a, lane);  // sum_{t >= lane} a_t
  float suf = __shfl_down(rs, 1, 64);         // sum_{t > lane} a_t
  if (lane == 63) suf = 0.f;
  d.cs[lane] = cs;
  d.dtp[lane] = dtp;
  d.W[lane] = __expf(suf) * dtp;
  if (lane == 63) {
    d.dch = __expf(cs);
    d.lsum += cs;
  }
}

// B^T operands of wave w: rows n = 32w + 16nb + c, k = j = 32m + 8g + s (from the LDS B rows).
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
__device__ __forceinline__ void state_update(const bf16_t* sB, const bf16_t* WXh, const bf16_t* WXl,
                                             f32x4 (&S)[8], float d, int w, int lane) {
  const int g = lane >> 4, c = lane & 15;
  u32x4 bt[2][2];
  load_bt_ops(sB, bt, w, lane);
#pragma unroll
  for (int t = 0; t < 8; ++t) S[t] *= d;
#pragma unroll
  for (int pb = 0; pb < 4; ++pb) {
    const int p = 16 * pb + c;
#pragma unroll
    for (int m = 0; m < 2; ++m) {
      const int off = off_pj(p, 32 * m + 8 * g);
      const bf16x8 bh = as_bf8(ld16(&WXh[off]));
      const bf16x8 bl = as_bf8(ld16(&WXl[off]));
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
                                                                SegPtrs sp, int H, int G) {
  __shared__ SmemState sm;
  const int nhb = H >> 1;
  const int seg = blockIdx.x / nhb;
  const int h0 = (blockIdx.x % nhb) * 2;
  const int4 si0 = sp.seg_info[seg];
  const int4 si = make_int4(uniform(si0.x), uniform(si0.y), uniform(si0.z), uniform(si0.w));
  const int nseg_seq = uniform(sp.seq_info[si.x].y);
  if (si.w == nseg_seq - 1) return;  // a sequence's last segment needs no local state
  const int tid = threadIdx.x, w = tid >> 6, lane = tid & 63;
  const int Di = H * kP;
  const uint32_t ld = (uint32_t)(Di + 2 * G * kN);
  const size_t boff = (size_t)Di + (size_t)(h0 / (H / G)) * kN;
  const float A = w < 2 ? __expf(a_log[h0 + w]) : 0.f;
  const float bias = w < 2 ? dt_bias[h0 + w] : 0.f;
  if (tid < 2) sm.d[tid].lsum = 0.f;

  f32x4 S[2][8];
#pragma unroll
  for (int hh = 0; hh < 2; ++hh)
#pragma unroll
    for (int t = 0; t < 8; ++t) S[hh][t] = f32x4{0.f, 0.f, 0.f, 0.f};

  PfB pb;
  PfX px[2];
  float pdt = 0.f;
  auto issue = [&](int q) {
    const int r0 = si.y + q * kQ;
    const int nr = min(kQ, si.z - q * kQ);
    const Rsrc rows = rows_rsrc(xbc + (size_t)r0 * ld, (uint32_t)nr * ld * 2u);
    load_b(pb, rows, ld, (uint32_t)boff);
    load_x(px[0], rows, ld, (uint32_t)(h0 * kP));
    load_x(px[1], rows, ld, (uint32_t)((h0 + 1) * kP));
    if (w < 2 && lane < nr) pdt = bf16_to_f32(dt[(size_t)(r0 + lane) * H + h0 + w]);
  };

  const int nchunks = (si.z + kQ - 1) / kQ;
  issue(0);
  for (int q = 0; q < nchunks; ++q) {
    const int nr = min(kQ, si.z - q * kQ);
    __syncthreads();  // the previous chunk is done with LDS
    store_b(sm.B, pb);
    if (w < 2) chunk_decay(sm.d[w], pdt, A, bias, nr, lane);
    __syncthreads();
    store_x<false>(nullptr, sm.WXh[0], sm.WXl[0], px[0], sm.d[0].W);
    store_x<false>(nullptr, sm.WXh[1], sm.WXl[1], px[1], sm.d[1].W);
    if (q + 1 < nchunks) issue(q + 1);
    __syncthreads();
    state_update(sm.B, sm.WXh[0], sm.WXl[0], S[0], sm.d[0].dch, w, lane);
    state_update(sm.B, sm.WXh[1], sm.WXl[1], S[1], sm.d[1].dch, w, lane);
  }
#pragma unroll
  for (int hh = 0; hh < 2; ++hh) {
    float* out = sp.seg_state + ((size_t)seg * H + h0 + hh) * (size_t)(kP * kN);
#pragma unroll
    for (int t = 0; t < 8; ++t) *reinterpret_cast<f32x4*>(out + state_elem(t, w, lane)) = S[hh][t];
  }
  if (tid < 2) sp.seg_decay[(size_t)seg * H + h0 + tid] = __expf(sm.d[tid].lsum);
}

// ---------------------------------------------------------------- outputs

__global__ __launch_bounds__(256, 2) void ssd_mfma_scan_kernel(
    bf16_t* __restrict__ y, const bf16_t* __restrict__ xbc, const bf16_t* __restrict__ dt,
    const float* __restrict__ a_log, const float* __restrict__ dt_bias, const float* __restrict__ Dp,
    float* __restrict__ pool, const int32_t* __restrict__ slots, SegPtrs sp, int H, int G) {
  __shared__ SmemScan sm;
  const int seg = blockIdx.x / H;
  const int h = blockIdx.x % H;
  const int4 si0 = sp.seg_info[seg];
  const int4 si = make_int4(uniform(si0.x), uniform(si0.y), uniform(si0.z), uniform(si0.w));
  const bool last = si.w == uniform(sp.seq_info[si.x].y) - 1;
  const int tid = threadIdx.x, w = tid >> 6, lane = tid & 63;
  const int g = lane >> 4, c = lane & 15;
  const int Di = H * kP;
  const uint32_t ld = (uint32_t)(Di + 2 * G * kN);
  const int grp = h / (H / G);
  const size_t boff = (size_t)Di + (size_t)grp * kN;
  const size_t coff = (size_t)Di + (size_t)G * kN + (size_t)grp * kN;
  const int irow = 16 * w + c;  // this lane's output row in the chunk
  const float A = __expf(a_log[h]), bias = dt_bias[h], dh = Dp[h];
  if (tid == 0) sm.d.lsum = 0.f;

  // the state entering the segment (written by the pass kernel)
  f32x4 S[8];
  {
    const float* in = sp.seg_state + ((size_t)seg * H + h) * (size_t)(kP * kN);
#pragma unroll
    for (int t = 0; t < 8; ++t) S[t] = *reinterpret_cast<const f32x4*>(in + state_elem(t, w, lane));
  }

  PfB pb;
  PfX px;
  u32x4 pc[4];
  float pdt = 0.f;
  auto issue = [&](int q) {
    const int r0 = si.y + q * kQ;
    const int nr = min(kQ, si.z - q * kQ);
    const Rsrc rows = rows_rsrc(xbc + (size_t)r0 * ld, (uint32_t)nr * ld * 2u);
    load_b(pb, rows, ld, (uint32_t)boff);
    load_x(px, rows, ld, (uint32_t)(h * kP));
    // C rows of this wave's row block: B-operand of G^T and of S C^T (k = n, col = i)
#pragma unroll
    for (int kk = 0; kk < 4; ++kk)
      pc[kk] = bld16(rows, 2u * ((uint32_t)irow * ld + (uint32_t)coff + (uint32_t)(32 * kk + 8 * g)));
    if (w == 0 && lane < nr) pdt = bf16_to_f32(dt[(size_t)(r0 + lane) * H + h]);
  };

  const int nchunks = (si.z + kQ - 1) / kQ;
  issue(0);
  for (int q = 0; q < nchunks; ++q) {
    const int r0 = si.y + q * kQ;
    const int nr = min(kQ, si.z - q * kQ);
    __syncthreads();  // (1) the previous chunk is done with LDS
    store_b(sm.B, pb);
    if (w == 0) chunk_decay(sm.d, pdt, A, bias, nr, lane);
    u32x4 cr[4];
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) cr[kk] = pc[kk];
    __syncthreads();  // (2) B rows and decay sums visible
    store_x<true>(sm.XT, sm.WXh, sm.WXl, px, sm.d.W);
    // S [p][n] in bf16 hi + lo halves
#pragma unroll
    for (int t = 0; t < 8; ++t) {
      const int p = 16 * (t & 3) + c;
      const int n = 32 * w + 16 * (t >> 2) + 4 * g;
      float lo[4];
#pragma unroll
      for (int r = 0; r < 4; ++r) lo[r] = S[t][r] - bf_round(S[t][r]);
      st8(&sm.Sh[off_pn(p, n)], u32x2{pk(S[t][0], S[t][1]), pk(S[t][2], S[t][3])});
      st8(&sm.Sl[off_pn(p, n)], u32x2{pk(lo[0], lo[1]), pk(lo[2], lo[3])});
    }
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
    if (q + 1 < nchunks) issue(q + 1);
    __syncthreads();  // (3) X^T, (w o X)^T and S tiles visible

    // ---- Y^T tiles (p block pb, i block w): exp(cs_i) S C^T + X^T M^T + D x ----
    const float csi = sm.d.cs[irow];
    const float ei = __expf(csi);
    f32x4 yacc[4];
#pragma unroll
    for (int pb4 = 0; pb4 < 4; ++pb4) {
      yacc[pb4] = f32x4{0.f, 0.f, 0.f, 0.f};
      const int p = 16 * pb4 + c;
#pragma unroll
      for (int kk = 0; kk < 4; ++kk) {
        const int off = off_pn(p, 32 * kk + 8 * g);
        yacc[pb4] = mfma(as_bf8(ld16(&sm.Sh[off])), as_bf8(cr[kk]), yacc[pb4]);
        yacc[pb4] = mfma(as_bf8(ld16(&sm.Sl[off])), as_bf8(cr[kk]), yacc[pb4]);
      }
      yacc[pb4] *= ei;
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
          const f32x4 csj = *reinterpret_cast<const f32x4*>(&sm.d.cs[j0]);
          const f32x4 dtj = *reinterpret_cast<const f32x4*>(&sm.d.dtp[j0]);
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
        for (int pb4 = 0; pb4 < 4; ++pb4) {
          const int p = 16 * pb4 + c;
          const u32x2 x0 = ld8(&sm.XT[off_pj(p, 32 * m + 4 * g)]);
          const u32x2 x1 = ld8(&sm.XT[off_pj(p, 32 * m + 16 + 4 * g)]);
          const bf16x8 xo = as_bf8(u32x4{x0.x, x0.y, x1.x, x1.y});
          yacc[pb4] = mfma(xo, as_bf8(mh), yacc[pb4]);
          yacc[pb4] = mfma(xo, as_bf8(ml), yacc[pb4]);
        }
        __builtin_amdgcn_sched_barrier(0);
      }
    }
    // + D x and store: lane holds y[i = irow][p = 16pb + 4g + r]; x from X^T
    {
      const Rsrc yrows = rows_rsrc(y + (size_t)r0 * Di, (uint32_t)nr * (uint32_t)Di * 2u);
#pragma unroll
      for (int pb4 = 0; pb4 < 4; ++pb4) {
        const int p0 = 16 * pb4 + 4 * g;
        float o[4];
#pragma unroll
        for (int r = 0; r < 4; ++r) o[r] = fmaf(dh, bf16_to_f32(sm.XT[off_pj(p0 + r, irow)]), yacc[pb4][r]);
        bst8(yrows, 2u * ((uint32_t)irow * (uint32_t)Di + (uint32_t)(h * kP + p0)),
             u32x2{pk(o[0], o[1]), pk(o[2], o[3])});
      }
    }
    // ---- state update ----
    state_update(sm.B, sm.WXh, sm.WXl, S, sm.d.dch, w, lane);
  }
  if (last) {
    float* out = pool + ((size_t)slots[si.x] * H + h) * (size_t)(kP * kN);
#pragma unroll
    for (int t = 0; t < 8; ++t) *reinterpret_cast<f32x4*>(out + state_elem(t, w, lane)) = S[t];
  }
}

}  // namespace

// Shapes the MFMA path covers: bf16, P = 64, N = 128, heads in pairs within one group (the
// state kernel takes two heads per workgroup), and 64-row offsets within 32 bits.
bool scan_mfma_supported(const mamba2_dims* d) {
  const int64_t Dc = (int64_t)d->nheads * d->headdim + 2 * (int64_t)d->ngroups * d->d_state;
  return d->act_dtype == MAMBA2_DTYPE_BF16 && d->headdim == kP && d->d_state == kN && d->nheads % 2 == 0 &&
         (d->nheads / d->ngroups) % 2 == 0 && Dc * kQ < ((int64_t)1 << 31);
}

hipError_t launch_scan_mfma(const ScanArgs& a, hipStream_t st) {
  const SegPtrs sp{(const int2*)(a.ws + a.lay.off_seq_info), (const int4*)(a.ws + a.lay.off_seg_info),
                   (float*)(a.ws + a.lay.off_seg_decay), (float*)(a.ws + a.lay.off_seg_state)};
  const mamba2_dims& d = a.dims;
  M2_LAUNCH("ssd_state", ssd_mfma_state_kernel, dim3((unsigned)(a.lay.nseg * (d.nheads / 2))), dim3(256), 0,
            st, (const bf16_t*)a.xbc, (const bf16_t*)a.dt, a.a_log, a.dt_bias, sp, d.nheads, d.ngroups);
  hipError_t e = launch_scan_pass(a, st);
  if (e != hipSuccess) return e;
  M2_LAUNCH("ssd_scan", ssd_mfma_scan_kernel, dim3((unsigned)(a.lay.nseg * d.nheads)), dim3(256), 0, st,
            (bf16_t*)a.y, (const bf16_t*)a.xbc, (const bf16_t*)a.dt, a.a_log, a.dt_bias, a.D, a.ssm_state,
            a.bd.slots, sp, d.nheads, d.ngroups);
  return hipSuccess;
}

}  // namespace m2
