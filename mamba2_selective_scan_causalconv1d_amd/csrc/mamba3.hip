// Mamba-3 SISO forward over packed variable-length sequences, for gfx950.
//
// The operator of "Mamba-3 SISO Long-Ragged Multi-Chunk Joint States Full VJP", section
// "What You Have", steps 1-7, per packed sequence and value head h:
//   qh_t, kh_t = rotary(q_t + q_bias[h], phi_t), rotary(k_t + k_bias[h], phi_t)  (one Q/K head
//               shared by the H value heads; pair a = components (2a, 2a+1) turned by phi_t[a])
//   phi_t[a]  = (sum_{s<=t} tanh(angles_s[a]) pi dt_s[h]) mod 2 pi
//   p = sigmoid(trap); sg_t = dt_{t+1} (1 - p_{t+1}) (0 at the sequence's last token);
//   scale_t = dt_t p_t + sg_t
//   y_t = sum_{s<=t} exp(sum_{r=s+1..t} adt_r) (qh_t . kh_s) scale_s v_s + d v_t - sg_t (qh_t . kh_t) v_t
//   out_t = y_t z_t sigmoid(z_t)
// and per sequence the final angle, the final state sum_s exp(sum_{r>s} adt_r) scale_s v_s kh_s^T,
// the last token's key kh and value v.
//
// Chunked form (64-row chunks, each within one sequence), with cs_i the sum of adt over the
// chunk's rows up to i and S_in the state entering the chunk:
//   y_i = sum_{j<=i} M_ij v_j + exp(cs_i) qh_i . S_in,
//   M_ij = (qh_i . kh_j) exp(cs_i - cs_j) scale_j (j < i),  M_ii = (qh_i . kh_i) dt_i p_i + d
//   (the diagonal folds the correction: scale_i - sg_i = dt_i p_i, and the skip d),
//   S_loc = sum_j exp(cs_last - cs_j) scale_j v_j kh_j^T,  S_in(next) = exp(cs_last) S_in + S_loc.
// Launches: chunk tables; per (chunk, head block) the chunk's rotary-angle totals and per
// (sequence, head) their running sums; per (chunk, head) the chunk state (and a sequence's
// finals); the state pass per (sequence, head); per (chunk group, head) the outputs, each
// workgroup walking its group's chunks with the next one's inputs fetched ahead.  The
// contractions (q.k over a chunk, the state's output term, M v and the chunk state) take fp32
// operands (the queries and keys after the bias and the rotation, M, the states, w v): each is
// split into bf16 hi and lo halves in LDS and multiplied as hi.hi + hi.lo + lo.hi on
// v_mfma_f32_16x16x32_bf16 (~2^-16 relative, well inside the output and state bars; v, exact
// in bf16, takes M's two halves directly).  The rotary angles entering each chunk are summed in
// double (their running sum covers whole sequences); within a chunk (at most 64 terms) in fp32.
#include <algorithm>
#include <initializer_list>

#include "common.h"

#include "../../include/mamba3.h"

namespace m2 {
namespace {

constexpr int kC = 64;       // chunk rows
constexpr int kMaxDK = 128;  // query / key width
constexpr int kMaxDV = 64;   // value width
constexpr int kMaxNA = 64;   // rotary pairs
constexpr int kBlock = 1024;  // threads of the chunk-state and output workgroups (16 waves)

__device__ __forceinline__ float bf(const bf16_t* p) { return bf16_to_f32(*p); }
__device__ __forceinline__ float sigmoidf_(float x) { return 1.f / (1.f + __expf(-x)); }
// Entries of the chunk and sequence tables at a wave-uniform index, read through the constant
// address space so that they are scalar loads: a vector load made uniform would wait for
// every vector load issued before it.
typedef const __attribute__((address_space(4))) int* ConstInts;
__device__ __forceinline__ int4 load_scalar(const int4* p, int i) {
  const ConstInts q = (ConstInts)p + 4 * i;
  return make_int4(q[0], q[1], q[2], q[3]);
}
__device__ __forceinline__ int2 load_scalar(const int2* p, int i) {
  const ConstInts q = (ConstInts)p + 2 * i;
  return make_int2(q[0], q[1]);
}
// A compiler-level fence: no memory access is moved across it (the loads before it are
// issued before those after it; waits are still placed only where values are used).
__device__ __forceinline__ void issue_order() { asm volatile("" ::: "memory"); }
// The rotary angles are summed in double: the running sum covers up to thousands of tokens,
// and fp32 rounding of its partial sums would add up to ~1e-4 radian.
constexpr double kTwoPiD = 6.283185307179586476925287;
constexpr double kPiD = 3.141592653589793238462643;
__device__ __forceinline__ double mod2pi(double x) {
  const double r = x - kTwoPiD * floor(x * (1.0 / kTwoPiD));
  return r < 0.0 ? r + kTwoPiD : (r >= kTwoPiD ? r - kTwoPiD : r);
}
// tanh from the hardware exponential and reciprocal: 1 - 2 / (e^{2|x|} + 1), absolute error
// ~1e-7 (what an angle needs), with the sign of x
__device__ __forceinline__ float tanh_fast(float x) {
  const float t = 1.f - 2.f * __builtin_amdgcn_rcpf(__expf(2.f * fabsf(x)) + 1.f);
  return copysignf(t, x);
}
// Inclusive prefix sum over the 64 lanes of a wave: shifts within 16-lane rows, then the row
// totals broadcast forward.  All 64 lanes must be active.
template <int kCtrl, int kRowMask>
__device__ __forceinline__ float dpp_add(float x) {
  return x + __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), kCtrl, kRowMask, 0xf, false));
}
__device__ __forceinline__ float wave_scan(float v) {
  v = dpp_add<0x111, 0xf>(v);  // row_shr:1
  v = dpp_add<0x112, 0xf>(v);  // row_shr:2
  v = dpp_add<0x114, 0xf>(v);  // row_shr:4
  v = dpp_add<0x118, 0xf>(v);  // row_shr:8
  v = dpp_add<0x142, 0xa>(v);  // row_bcast:15
  return dpp_add<0x143, 0xc>(v);  // row_bcast:31
}

typedef float f32x4 __attribute__((ext_vector_type(4)));
// The bf16 form of an fp32 product: each fp32 operand split into a bf16 hi and lo half
// (x = hi + lo to ~2^-17), the product taken as hi.hi + hi.lo + lo.hi on v_mfma_f32_16x16x32_bf16
// (the dropped lo.lo term is ~2^-16 of it): three instructions of ~16 cycles for 8192
// multiply-adds, against eight fp32 16x16x4 ones of ~47.  Operand layout: lane l supplies row
// (A) or column (B) l % 16 and eight consecutive k, 8 (l / 16) .. + 7, of a 32-wide k step; the
// result layout is the fp32 instruction's (register r of lane l: D[4 (l / 16) + r][l % 16]).
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
__device__ __forceinline__ f32x4 mfma_bf(const u32x4& a, const u32x4& b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a), __builtin_bit_cast(bf16x8, b), c, 0, 0,
                                                  0);
}
__device__ __forceinline__ f32x4 mfma3(const u32x4& ah, const u32x4& al, const u32x4& bh, const u32x4& bl, f32x4 c) {
  c = mfma_bf(ah, bh, c);
  c = mfma_bf(ah, bl, c);
  return mfma_bf(al, bh, c);
}
__device__ __forceinline__ u32x4 lds16(const bf16_t* p) { return *reinterpret_cast<const u32x4*>(p); }
// hi and lo halves of x, each rounded to nearest even
__device__ __forceinline__ uint32_t bf_hi(float x) { return f32_to_bf16(x); }
__device__ __forceinline__ uint32_t bf_lo(float x, uint32_t hi) { return f32_to_bf16(x - bf16_to_f32(hi)); }

struct M3Ptrs {
  const bf16_t* q;
  const bf16_t* k;
  const bf16_t* v;
  const float* adt;
  const float* dt;
  const bf16_t* trap;
  const float* q_bias;
  const float* k_bias;
  const bf16_t* angles;
  const float* d;
  const bf16_t* z;
  bf16_t* out;
  bf16_t* fin_angle;
  float* fin_ssm;
  float* fin_k;
  bf16_t* fin_v;
  const int2* seq_info;   // [S] (first chunk, chunks)
  const int4* chunk_info;  // [nch] (sequence, first row, rows, index in sequence)
  float* ang_tot;         // [nch][H][NA] sum over the chunk of tanh(angles) pi dt, then the angle entering the chunk
  float* decay;           // [nch][H] exp(sum of adt over the chunk)
  float* state;           // [nch][H][DV][DK]: at chunk c + 1 the local state of chunk c, then S_in(c + 1)
  int H, DK, DV, NA;
  int T;  // rows of the batch
};

// ------------------------------------------------------------------ rotary-angle totals

// grid (chunk, head block of kAngHeads), 256 threads: theta = tanh(angles) pi for the chunk's
// rows and the block's dt in LDS; then per (head, pair) the chunk's sum of theta dt, in double,
// stored reduced into [0, 2 pi).  kTables (at most 256 sequences): each workgroup finds its
// chunk from the row offsets and the first one stores the chunk tables for the later launches.
constexpr int kAngHeads = 8;
template <bool kTables>
__global__ __launch_bounds__(256) void m3_angle_totals_kernel(M3Ptrs P, int nch, const int32_t* __restrict__ cu,
                                                              int S, int2* __restrict__ seq_out,
                                                              int4* __restrict__ chunk_out) {
  __shared__ float sTh[kC][kMaxNA + 1];
  __shared__ float sDt[kC][65];
  const int c = blockIdx.x;
  if (c >= nch) return;  // uniform over the workgroup
  const int4 ci = kTables ? own_segment<256>(cu, S, kC, c, seq_out, chunk_out, blockIdx.x == 0 && blockIdx.y == 0)
                          : P.chunk_info[c];
  for (int e = threadIdx.x; e < kC * P.NA; e += blockDim.x) {
    const int j = e / P.NA, a = e - j * P.NA;
    sTh[j][a] = j < ci.z ? tanhf(bf(P.angles + (size_t)(ci.y + j) * P.NA + a)) : 0.f;
  }
  {
    const int h0 = blockIdx.y * kAngHeads;
    const int nh = min(kAngHeads, P.H - h0);
    __syncthreads();
    for (int e = threadIdx.x; e < kC * nh; e += blockDim.x) {
      const int j = e / nh, hh = e - j * nh;
      sDt[j][hh] = j < ci.z ? P.dt[(size_t)(ci.y + j) * P.H + h0 + hh] : 0.f;
    }
    __syncthreads();
    for (int e = threadIdx.x; e < nh * P.NA; e += blockDim.x) {
      const int hh = e / P.NA, a = e - hh * P.NA;
      double acc = 0.0;
      for (int j = 0; j < ci.z; ++j) acc += (double)sTh[j][a] * (double)sDt[j][hh];
      P.ang_tot[((size_t)c * P.H + h0 + hh) * P.NA + a] = (float)mod2pi(acc * kPiD);
    }
  }
}

// grid (sequence, (head, pair) blocks), 256 threads: per (head, pair), the rotary angle entering
// each chunk of the sequence (the sum of the earlier chunks' totals, mod 2 pi), in place of the
// totals.  The totals are loaded four chunks at a time.
__global__ __launch_bounds__(256) void m3_angle_prefix_kernel(M3Ptrs P, int S) {
  const int s = blockIdx.x;
  const int e = blockIdx.y * blockDim.x + threadIdx.x;
  if (s >= S || e >= P.H * P.NA) return;
  const int2 si = P.seq_info[s];
  double acc = 0.0;
  for (int k0 = 0; k0 < si.y; k0 += 4) {
    float t[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) t[i] = k0 + i < si.y ? P.ang_tot[(size_t)(si.x + k0 + i) * P.H * P.NA + e] : 0.f;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      if (k0 + i < si.y) {
        P.ang_tot[(size_t)(si.x + k0 + i) * P.H * P.NA + e] = (float)acc;
        acc = mod2pi(acc + (double)t[i]);
      }
    }
  }
}

// ------------------------------------------------------------------ chunk rows

// Per-row scalars of a chunk for head h and its rotary angles, in LDS:
//   cs[i] = sum of adt over rows <= i of the chunk; sc[i] = scale_i; dp[i] = dt_i p_i;
//   phi[i][a] = the rotary angle of row i, pair a, and its cosine and sine.
// kCS: the rotation kept as cos and sin (for two rotations of the same rows), else the angle.
template <bool kCS>
struct RowLds;
template <>
struct RowLds<false> {
  float cs[kC], sc[kC], dp[kC];
  float phi[kC][kMaxNA];
};
template <>
struct RowLds<true> {
  float cs[kC], sc[kC], dp[kC];
  float cosv[kC][kMaxNA], sinv[kC][kMaxNA];
};


// The loads of the row scalars and angles, issued on their own so that a caller can order them
// against other loads (a wave waits for its loads in issue order), at addresses clamped into
// the chunk and the batch, with no branch around a load and no use of a loaded value here: a
// guarded load would be waited for inside its branch, and a select right after a load waits
// for it.  The values are raw; rows_from keeps those of valid rows.  The next row's dt and trap
// are fetched wherever the batch has that row; they are used only where it belongs to the same
// sequence.
// kIt: rotary pairs per wave the caller covers (NA <= kIt * kBlock / 64).
template <int kIt>
struct RowFetch {
  float dt, adt, dtn;
  bf16_t trap, trapn;
  float base_f[kIt];
  bf16_t ang[kIt];
};
template <int kIt>
__device__ __forceinline__ void fetch_row_scalars(RowFetch<kIt>& f, const M3Ptrs& P, int c, const int4& ci, int h) {
  const int tid = threadIdx.x, w = tid >> 6, lane = tid & 63, nw = blockDim.x >> 6;
  const int r = ci.y + min(lane, ci.z - 1);  // a row of the chunk for every lane
  const int rn = min(r + 1, P.T - 1);
  f.dt = P.dt[(size_t)r * P.H + h];
  f.adt = P.adt[(size_t)r * P.H + h];  // these four for wave 0 only, fetched by every wave
  f.trap = P.trap[(size_t)r * P.H + h];
  f.dtn = P.dt[(size_t)rn * P.H + h];
  f.trapn = P.trap[(size_t)rn * P.H + h];
  if (P.NA > 0) {
#pragma unroll
    for (int it = 0; it < kIt; ++it) {
      const int ac = min(w + it * nw, P.NA - 1);
      f.base_f[it] = P.ang_tot[((size_t)c * P.H + h) * P.NA + ac];
      f.ang[it] = P.angles[(size_t)r * P.NA + ac];
    }
  }
}
// The row scalars and angles from the fetched values, into L:
//   cs[i] = sum of adt over rows <= i of the chunk; sc[i] = scale_i; dp[i] = dt_i p_i;
//   the rotary angle of row i, pair a: the angle entering the chunk (the prefix kernel's), then
//   the running sum over this chunk's rows (at most 64 terms: fp32, by DPP), reduced mod 2 pi in
//   double; kept as its cosine and sine (kCS) or as the angle.
template <bool kCS, int kIt>
__device__ __forceinline__ void rows_from(const RowFetch<kIt>& f, const M3Ptrs& P, const int4& ci, const int2& si,
                                          RowLds<kCS>& L) {
  const int tid = threadIdx.x, w = tid >> 6, nw = blockDim.x >> 6;
  int lane = tid & 63;
  asm volatile("" : "+v"(lane));  // the table addresses are recomputed here, not kept live across a caller's loop
  const bool on = lane < ci.z;
  const float dtv = on ? f.dt : 0.f;
  if (w == 0) {
    // decay prefix, p, scale (the next row may lie in the next chunk of the same sequence)
    const float cs = wave_scan(on ? f.adt : 0.f);
    const bool last_chunk = ci.w == si.y - 1;
    const bool has_next = on && (lane + 1 < ci.z || !last_chunk);
    const float p = on ? sigmoidf_(bf16_to_f32(f.trap)) : 0.f;
    float sg = 0.f;
    if (has_next) {
      const float pn = sigmoidf_(bf16_to_f32(f.trapn));
      sg = f.dtn * (1.f - pn);
    }
    L.cs[lane] = cs;
    L.sc[lane] = dtv * p + sg;
    L.dp[lane] = dtv * p;
  }
#pragma unroll
  for (int it = 0; it < kIt; ++it) {
    const int a = w + it * nw;
    if (a >= P.NA) break;
    const float v = wave_scan(on ? tanh_fast(bf16_to_f32(f.ang[it])) * (float)kPiD * dtv : 0.f);
    const float ph = (float)mod2pi((double)f.base_f[it] + (double)v);
    if constexpr (kCS) {
      L.cosv[lane][a] = __cosf(ph);
      L.sinv[lane][a] = __sinf(ph);
    } else {
      L.phi[lane][a] = ph;
    }
  }
}

// dst = rotary(src_i + bias, phi_i) for the chunk's rows (zeros past its end), fp32: row i at
// dst[i * ld + n], or transposed (kT) at dst[n * ld + i].  One thread per (row, component pair).
__device__ __forceinline__ int pad32(int n) { return (n + 31) & ~31; }
// The chunk's rows of a [T, DK] bf16 input and a head's bias, as kBlock threads stage them: each
// thread holds kRowIt (row, component pair) units, fetched with every load in flight at once.
constexpr int kRowIt = kC * (kMaxDK / 2) / kBlock;
struct RowUnits {
  uint32_t raw[kRowIt];
  float2 bias[kRowIt];
};
// np: component pairs per row of the staging (DK / 2, or more for zero padding); unit e is
// row e / np, pair e % np (fetch_raw and fetch_bias below).
// rotary(src_i + bias, phi_i) from the fetched units, as bf16 hi and lo planes [i * ld + n]
// (zeros past the chunk's end and, along the width, up to the next multiple of 32).
// raw: the fetched pairs (fetch_raw); bias: the head's bias, DK floats (in LDS).
__device__ __forceinline__ void rotate_rows(const uint32_t (&raw)[kRowIt], const float* bias, const RowLds<true>& L,
                                            const int4& ci, int DK, int NA, bf16_t* dh, bf16_t* dl, int ld) {
  const int npair = DK / 2, np = pad32(DK) / 2, nfill = kC * np;  // np as in the fetch
#pragma unroll
  for (int it = 0; it < kRowIt; ++it) {
    const int e = (int)threadIdx.x + it * kBlock;
    if (e >= nfill) break;
    const int i = e / np, a = e - i * np;
    float x0 = 0.f, x1 = 0.f;
    if (i < ci.z && a < npair) {
      const uint32_t two = raw[it];
      const float2 b = *reinterpret_cast<const float2*>(bias + 2 * a);
      x0 = bf16_to_f32(two & 0xffffu) + b.x;
      x1 = bf16_to_f32(two >> 16) + b.y;
      if (a < NA) {
        const float cs = L.cosv[i][a], sn = L.sinv[i][a];
        const float r0 = x0 * cs - x1 * sn, r1 = x0 * sn + x1 * cs;
        x0 = r0;
        x1 = r1;
      }
    }
    const uint32_t h0 = bf_hi(x0), h1 = bf_hi(x1);
    *reinterpret_cast<uint32_t*>(dh + i * ld + 2 * a) = h0 | (h1 << 16);
    *reinterpret_cast<uint32_t*>(dl + i * ld + 2 * a) = bf_lo(x0, h0) | (bf_lo(x1, h1) << 16);
  }
}
// Transposed staging in row pairs: unit e is rows 2 (e / npair) and + 1, component pair
// e % npair, so that each plane takes one 4-byte store per unit and column.  u.raw[2 it + r]
// holds row 2 ip + r of unit it (raw: rows past the chunk's end hold its last row's values);
// u.bias[it] the pair's bias.
__device__ __forceinline__ void fetch_rows_t(RowUnits& u, const bf16_t* src, const float* bias, const int4& ci,
                                             int DK) {
  const int npair = DK / 2;
#pragma unroll
  for (int it = 0; it < kRowIt / 2; ++it) {
    const int e = (int)threadIdx.x + it * kBlock, ip = e / npair, a = e - ip * npair;
#pragma unroll
    for (int r = 0; r < 2; ++r) {
      const int i = 2 * ip + r;  // loaded at a row clamped into the chunk (used for rows of it only)
      u.raw[2 * it + r] = *reinterpret_cast<const uint32_t*>(src + (size_t)(ci.y + min(i, ci.z - 1)) * DK + 2 * a);
    }
    u.bias[it] = *reinterpret_cast<const float2*>(bias + 2 * a);
  }
}
// kh^T as hi and lo planes [n][j] (zeros past the chunk's end) from fetch_rows_t's units; fin
// (may be null): the fp32 values of row il.
__device__ __forceinline__ void rotate_rows_t(const RowUnits& u, const RowLds<false>& L, const int4& ci, int DK, int NA, bf16_t* dh,
                              bf16_t* dl, int ld, float* fin, int il) {
  const int npair = DK / 2, n = (kC / 2) * npair;
#pragma unroll
  for (int it = 0; it < kRowIt / 2; ++it) {
    const int e = (int)threadIdx.x + it * kBlock;
    if (e >= n) break;
    const int ip = e / npair, a = e - ip * npair;
    uint32_t hp[2] = {0u, 0u}, lp[2] = {0u, 0u};  // planes of components 2a, 2a + 1: rows 2 ip, 2 ip + 1
#pragma unroll
    for (int r = 0; r < 2; ++r) {
      const int i = 2 * ip + r;
      float x0 = 0.f, x1 = 0.f;
      if (i < ci.z) {
        const uint32_t two = u.raw[2 * it + r];
        x0 = bf16_to_f32(two & 0xffffu) + u.bias[it].x;
        x1 = bf16_to_f32(two >> 16) + u.bias[it].y;
        if (a < NA) {
          const float sn = __sinf(L.phi[i][a]), cs = __cosf(L.phi[i][a]);
          const float r0 = x0 * cs - x1 * sn, r1 = x0 * sn + x1 * cs;
          x0 = r0;
          x1 = r1;
        }
        if (fin && i == il) {
          fin[2 * a] = x0;
          fin[2 * a + 1] = x1;
        }
      }
      const uint32_t h0 = bf_hi(x0), h1 = bf_hi(x1);
      hp[0] |= h0 << (16 * r);
      hp[1] |= h1 << (16 * r);
      lp[0] |= bf_lo(x0, h0) << (16 * r);
      lp[1] |= bf_lo(x1, h1) << (16 * r);
    }
    *reinterpret_cast<uint32_t*>(dh + (2 * a) * ld + 2 * ip) = hp[0];
    *reinterpret_cast<uint32_t*>(dh + (2 * a + 1) * ld + 2 * ip) = hp[1];
    *reinterpret_cast<uint32_t*>(dl + (2 * a) * ld + 2 * ip) = lp[0];
    *reinterpret_cast<uint32_t*>(dl + (2 * a + 1) * ld + 2 * ip) = lp[1];
  }
}
// The chunk's rows of head h's values in row pairs: unit e is rows 2 (e / DV) and + 1, column
// e % DV (vv[2 it + r]: row 2 jp + r; raw: rows past the chunk's end hold its last row's values).
constexpr int kValIt = kC * kMaxDV / kBlock;
__device__ __forceinline__ void fetch_values_t(bf16_t (&vv)[kValIt], const M3Ptrs& P, const int4& ci, int h) {
#pragma unroll
  for (int it = 0; it < kValIt / 2; ++it) {
    const int e = (int)threadIdx.x + it * kBlock, jp = e / P.DV, f = e - jp * P.DV;
#pragma unroll
    for (int r = 0; r < 2; ++r) {
      const int j = 2 * jp + r;  // loaded at a row clamped into the chunk (used for rows of it only)
      vv[2 * it + r] = P.v[((size_t)(ci.y + min(j, ci.z - 1)) * P.H + h) * P.DV + f];
    }
  }
}
// A chunk's queries and keys (raw pairs, in rotate_rows' unit order; the biases are the head's
// and fetched once), values (fetch_values_t's order) and entering state, in registers, as
// loaded (no select: each use keeps the valid entries).
struct ChunkData {
  uint32_t q[kRowIt], k[kRowIt];
  bf16_t v[kValIt];
  float4 s[kMaxDV * kMaxDK / 4 / kBlock];
};
__device__ __forceinline__ void fetch_raw(uint32_t (&raw)[kRowIt], const bf16_t* src, const int4& ci, int DK, int np) {
  const int npair = DK / 2;
#pragma unroll
  for (int it = 0; it < kRowIt; ++it) {
    const int e = (int)threadIdx.x + it * kBlock, i = e / np, a = e - i * np;
    // loaded at a row and pair clamped into the chunk (rotate_rows uses units of it only)
    raw[it] = *reinterpret_cast<const uint32_t*>(src + (size_t)(ci.y + min(i, ci.z - 1)) * DK + 2 * min(a, npair - 1));
  }
}
__device__ __forceinline__ void fetch_chunk(ChunkData& d, const M3Ptrs& P, int c, const int4& ci, int h, int np) {
  fetch_raw(d.q, P.q, ci, P.DK, np);
  fetch_raw(d.k, P.k, ci, P.DK, np);
  fetch_values_t(d.v, P, ci, h);
  const int n4s = P.DV * (P.DK / 4);
  const float4* sin = reinterpret_cast<const float4*>(P.state + ((size_t)c * P.H + h) * (size_t)P.DV * P.DK);
  // every chunk's slot lies in the workspace (a sequence's first chunk's is not written: its
  // values are loaded and not used)
#pragma unroll
  for (int it = 0; it < kMaxDV * kMaxDK / 4 / kBlock; ++it) d.s[it] = sin[min((int)threadIdx.x + it * kBlock, n4s - 1)];
}

// ------------------------------------------------------------------ chunk states

constexpr int kLdB = kMaxDK + 8;  // LDS row pitch of query / key / state rows (bf16 elements)
constexpr int kLdT = kC + 8;      // LDS row pitch of transposed tiles (a chunk's rows along a row)

// grid (chunk, head), kBlock threads: S_loc = sum_j exp(cs_last - cs_j) scale_j v_j kh_j^T, stored
// at chunk c + 1 (the sequence's last chunk: in the final-state output, which the pass then
// completes); the chunk's decay factor; for a sequence's last chunk, its final K, V and angle.
// S_loc [DV][DK] = (w o V)^T K on 16 x 16 tiles dealt over the waves, the chunk's rows as k
// (two 32-row steps), both operands transposed in LDS as bf16 hi / lo planes.
// KDK, KDV: the query / key and value widths when fixed at compile time (the address
// arithmetic then has no run-time divisions), else 0; KNA: the most rotary pairs covered (64
// when the widths are not fixed).
template <int KDK, int KDV, int KNA>
__global__ __launch_bounds__(kBlock) void m3_chunk_state_kernel(M3Ptrs P, int nch) {
  if constexpr (KDK != 0) {
    P.DK = KDK;
    P.DV = KDV;
  }
  __shared__ __attribute__((aligned(16))) bf16_t sKt[2][kMaxDK * kLdT];  // kh^T [n][j], hi and lo
  __shared__ __attribute__((aligned(16))) bf16_t sVt[2][kMaxDV * kLdT];  // (w v)^T [e][j], hi and lo
  __shared__ RowLds<false> L;
  const int c = blockIdx.x, h = blockIdx.y;
  if (c >= nch) return;
  const int4 ci = P.chunk_info[c];
  const int2 si = P.seq_info[ci.x];
  const bool last = ci.w == si.y - 1;
  // the row scalars' loads, then the chunk's keys and values, then the row scalars' arithmetic
  // (which waits for its own loads only)
  RowFetch<(KNA + kBlock / 64 - 1) / (kBlock / 64)> rf;
  fetch_row_scalars(rf, P, c, ci, h);
  RowUnits ku;
  fetch_rows_t(ku, P.k, P.k_bias + (size_t)h * P.DK, ci, P.DK);
  bf16_t vv[kValIt];
  fetch_values_t(vv, P, ci, h);
  rows_from(rf, P, ci, si, L);
  __syncthreads();
  const int il = ci.z - 1;
  rotate_rows_t(ku, L, ci, P.DK, P.NA, sKt[0], sKt[1], kLdT, last ? P.fin_k + ((size_t)ci.x * P.H + h) * P.DK : nullptr,
                il);
  const float cl = L.cs[il];
#pragma unroll
  for (int it = 0; it < kValIt / 2; ++it) {
    const int e = (int)threadIdx.x + it * kBlock, jp = e / P.DV, f = e - jp * P.DV;
    if (e >= (kC / 2) * P.DV) break;
    uint32_t hp = 0u, lp = 0u;
#pragma unroll
    for (int r = 0; r < 2; ++r) {
      const int j = 2 * jp + r;
      const float val = j < ci.z ? bf16_to_f32(vv[2 * it + r]) * (__expf(cl - L.cs[j]) * L.sc[j]) : 0.f;
      const uint32_t hi = bf_hi(val);
      hp |= hi << (16 * r);
      lp |= bf_lo(val, hi) << (16 * r);
    }
    *reinterpret_cast<uint32_t*>(sVt[0] + f * kLdT + 2 * jp) = hp;
    *reinterpret_cast<uint32_t*>(sVt[1] + f * kLdT + 2 * jp) = lp;
  }
  __syncthreads();
  const int w = threadIdx.x >> 6, lane = threadIdx.x & 63, lr = lane & 15, lg = lane >> 4;
  const int ne = P.DV / 16, nn = P.DK / 16;
  float* dst = last ? P.fin_ssm + ((size_t)ci.x * P.H + h) * (size_t)P.DV * P.DK
                    : P.state + ((size_t)(c + 1) * P.H + h) * (size_t)P.DV * P.DK;
  // both 32-row steps (rows past the chunk's end are zero in both operands)
  for (int t = w; t < ne * nn; t += (int)(blockDim.x >> 6)) {
    const int eb = t / nn, nb = t - eb * nn;
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int ks = 0; ks < kC / 32; ++ks) {
      const int ao = (eb * 16 + lr) * kLdT + 32 * ks + 8 * lg, bo = (nb * 16 + lr) * kLdT + 32 * ks + 8 * lg;
      acc = mfma3(lds16(sVt[0] + ao), lds16(sVt[1] + ao), lds16(sKt[0] + bo), lds16(sKt[1] + bo), acc);
    }
#pragma unroll
    for (int r = 0; r < 4; ++r) dst[(size_t)(eb * 16 + 4 * lg + r) * P.DK + nb * 16 + lr] = acc[r];
  }
  if (threadIdx.x == 0) P.decay[(size_t)c * P.H + h] = __expf(cl);
  if (last) {
    for (int f = threadIdx.x; f < P.DV; f += blockDim.x)
      P.fin_v[((size_t)ci.x * P.H + h) * P.DV + f] = P.v[((size_t)(ci.y + il) * P.H + h) * P.DV + f];
    for (int a2 = threadIdx.x; a2 < P.NA; a2 += blockDim.x)
      P.fin_angle[((size_t)ci.x * P.H + h) * P.NA + a2] = (bf16_t)f32_to_bf16(L.phi[il][a2]);
  }
}

// ------------------------------------------------------------------ state pass

// One thread per float4 of a head's state, per sequence (strided over grid z): S_in(0) = 0;
// S_in(c + 1) = dec(c) S_in(c) + S_loc(c) written over S_loc(c) at chunk c + 1; the final
// state = dec(last) S_in(last) + S_loc(last), completed in place in the final-state output.
__global__ __launch_bounds__(256) void m3_pass_kernel(M3Ptrs P, int S) {
  const int f = blockIdx.x * blockDim.x + threadIdx.x;
  const int h = blockIdx.y;
  const int f4 = P.DV * P.DK / 4;
  if (f >= f4) return;
  for (int s = blockIdx.z; s < S; s += gridDim.z) {
    const int2 si = P.seq_info[s];
    float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
    auto at = [&](int k) -> float4* {  // chunk k's local state, where S_in of chunk k + 1 goes
      const int c = si.x + k;
      return k + 1 < si.y ? reinterpret_cast<float4*>(P.state + ((size_t)(c + 1) * P.H + h) * (size_t)P.DV * P.DK)
                          : reinterpret_cast<float4*>(P.fin_ssm + ((size_t)s * P.H + h) * (size_t)P.DV * P.DK);
    };
    // the local states and decays of kBatchM chunks are loaded before the chain runs through them
    constexpr int kBatchM = 8;
    for (int k0 = 0; k0 < si.y; k0 += kBatchM) {
      float4 l[kBatchM];
      float dec[kBatchM];
#pragma unroll
      for (int i = 0; i < kBatchM; ++i) {
        const int k = k0 + i;
        dec[i] = k < si.y ? P.decay[(size_t)(si.x + k) * P.H + h] : 0.f;
        l[i] = k < si.y ? at(k)[f] : make_float4(0.f, 0.f, 0.f, 0.f);
      }
#pragma unroll
      for (int i = 0; i < kBatchM; ++i) {
        if (k0 + i >= si.y) break;
        acc = make_float4(fmaf(dec[i], acc.x, l[i].x), fmaf(dec[i], acc.y, l[i].y), fmaf(dec[i], acc.z, l[i].z),
                          fmaf(dec[i], acc.w, l[i].w));
        at(k0 + i)[f] = acc;
      }
    }
  }
}

// ------------------------------------------------------------------ outputs

// grid (chunk group, head), kBlock threads (four waves per SIMD at one workgroup per CU, which
// the LDS allows).  Workgroup (b, h) takes chunks b, b + gridDim.x, ... of head h; the next
// chunk's queries, keys, values and entering state are fetched into registers while the current
// one is computed (its own row scalars and gate inputs are fetched first, so that waiting for
// them never waits for the prefetch).  Per chunk: (1) rotated queries and keys in LDS (rows,
// bf16 hi / lo planes, zero-padded to a multiple of 32 columns), the values transposed (bf16,
// exact); (2) G = qh kh^T on the ten lower-triangular 16 x 16 tiles, turned into M
// (exp(cs_i - cs_j) scale_j below the diagonal, dt_i p_i and d on it; the tiles above are zero),
// in LDS as hi / lo planes; (3) the state entering the chunk over the keys' LDS, as hi / lo
// planes; (4) Y = exp(cs_i) qh S_in^T + M v on 16 x 16 tiles (rows x value columns), one per
// wave, the gate, bf16 stores.
// KDK, KDV: the query / key and value widths when fixed at compile time (the address
// arithmetic then has no run-time divisions and the k steps are unrolled), else 0; KNA: the
// most rotary pairs covered (64 when the widths are not fixed).
template <int KDK, int KDV, int KNA>
__global__ __launch_bounds__(kBlock) void m3_chunk_out_kernel(M3Ptrs P, int nch) {
  if constexpr (KDK != 0) {
    P.DK = KDK;
    P.DV = KDV;
  }
  __shared__ __attribute__((aligned(16))) bf16_t sQ[2][kC * kLdB];     // qh [i][n], hi and lo
  __shared__ __attribute__((aligned(16))) bf16_t sKS[2][kC * kLdB];    // kh [j][n], then S_in [e][n]
  __shared__ __attribute__((aligned(16))) bf16_t sVt[kMaxDV * kLdT];   // v^T [e][j]
  __shared__ __attribute__((aligned(16))) bf16_t sM[2][kC * kLdT];     // M [i][j], hi and lo
  __shared__ RowLds<true> L;
  __shared__ __attribute__((aligned(16))) float sBias[2][kMaxDK];        // the head's q and k biases
  const int h = blockIdx.y, stride = (int)gridDim.x;
  int c = blockIdx.x;
  if (c >= nch) return;
  const int npad = pad32(P.DK) / 2;  // component pairs per staged row, zero padding included
  const int w = threadIdx.x >> 6, lane = threadIdx.x & 63, lr = lane & 15, lg = lane >> 4;
  const int nwv = blockDim.x >> 6;
  const float dh = P.d[h];
  for (int e = threadIdx.x; e < 2 * P.DK; e += blockDim.x)  // visible after the loop's first barrier
    sBias[e / P.DK][e % P.DK] = (e < P.DK ? P.q_bias : P.k_bias)[(size_t)h * P.DK + e % P.DK];
  // the wave's output tile of a chunk (16 waves cover its at most 4 x 4 tiles) and its gate
  // inputs, loaded at rows clamped into the chunk (only rows of it are stored)
  const int nks = pad32(P.DK) / 32;
  const int neb = P.DV / 16;
  auto fetch_gate = [&](float (&zf)[4], const int4& cq) {
    const int tb = w / neb, te = w - tb * neb;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int i = tb * 16 + 4 * lg + r;
      zf[r] = bf(P.z + ((size_t)(cq.y + min(i, cq.z - 1)) * P.H + h) * P.DV + te * 16 + lr);
    }
  };
  int4 ci = load_scalar(P.chunk_info, c);
  int2 si = load_scalar(P.seq_info, ci.x);
  RowFetch<(KNA + kBlock / 64 - 1) / (kBlock / 64)> rf;
  fetch_row_scalars(rf, P, c, ci, h);
  float zf[4];
  fetch_gate(zf, ci);
  issue_order();
  ChunkData cur;
  fetch_chunk(cur, P, c, ci, h, npad);
  int cn = c + stride;
  int4 cin = load_scalar(P.chunk_info, min(cn, nch - 1));
  // the tiles of M above the diagonal are zero for every chunk
  for (int e = threadIdx.x; e < kC * kC; e += blockDim.x) {
    const int i = e / kC, j = e - i * kC;
    if ((j >> 4) > (i >> 4)) {
      sM[0][i * kLdT + j] = (bf16_t)0;
      sM[1][i * kLdT + j] = (bf16_t)0;
    }
  }
  for (;;) {
    const int nib = (ci.z + 15) / 16;  // 16-row blocks holding rows of the chunk
    const bool has_tile = w < nib * neb;
    const int tib = w / neb, teb = w - tib * neb;
    const int f = teb * 16 + lr;
    // the next chunk's data (this chunk's again when there is none, so the loads stay
    // unconditional), issued after this chunk's row scalars and gate inputs, so that waiting
    // for those never waits for the prefetch
    const bool more = cn < nch;
    const int cl = more ? cn : c;
    const int4 cil = more ? cin : ci;
    issue_order();
    ChunkData nxt;
    fetch_chunk(nxt, P, cl, cil, h, npad);
    issue_order();
    const int2 sil = load_scalar(P.seq_info, cil.x);
    const int cnn = cn + stride;
    const int4 cinn = load_scalar(P.chunk_info, min(cnn, nch - 1));

    rows_from(rf, P, ci, si, L);
    __syncthreads();
    rotate_rows(cur.q, sBias[0], L, ci, P.DK, P.NA, sQ[0], sQ[1], kLdB);
    rotate_rows(cur.k, sBias[1], L, ci, P.DK, P.NA, sKS[0], sKS[1], kLdB);
#pragma unroll
    for (int it = 0; it < kValIt / 2; ++it) {
      const int e = (int)threadIdx.x + it * kBlock, jp = e / P.DV, fv = e - jp * P.DV;
      if (e >= (kC / 2) * P.DV) break;
      const uint32_t v0 = 2 * jp < ci.z ? cur.v[2 * it] : 0u, v1 = 2 * jp + 1 < ci.z ? cur.v[2 * it + 1] : 0u;
      *reinterpret_cast<uint32_t*>(sVt + fv * kLdT + 2 * jp) = v0 | (v1 << 16);
    }
    __syncthreads();
    // M on the lower-triangular tiles (ib, jb), jb <= ib; tiles dealt round robin over the waves
    for (int t = w; t < 10; t += nwv) {
      const int ib = t < 1 ? 0 : t < 3 ? 1 : t < 6 ? 2 : 3;
      const int jb = t - ib * (ib + 1) / 2;
      f32x4 g = {0.f, 0.f, 0.f, 0.f};
      if (ib < nib) {
        for (int ks = 0; ks < nks; ++ks) {
          const int ao = (ib * 16 + lr) * kLdB + 32 * ks + 8 * lg, bo = (jb * 16 + lr) * kLdB + 32 * ks + 8 * lg;
          g = mfma3(lds16(sQ[0] + ao), lds16(sQ[1] + ao), lds16(sKS[0] + bo), lds16(sKS[1] + bo), g);
        }
      }
      const int j = jb * 16 + lr;
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int i = ib * 16 + 4 * lg + r;
        float m = 0.f;
        if (j < i) m = g[r] * __expf(L.cs[i] - L.cs[j]) * L.sc[j];
        else if (j == i) m = fmaf(g[r], L.dp[i], dh);
        const uint32_t hi = bf_hi(m);
        sM[0][i * kLdT + j] = (bf16_t)hi;
        sM[1][i * kLdT + j] = (bf16_t)bf_lo(m, hi);
      }
    }
    __syncthreads();  // M complete; the keys are no longer read
    const bool has_in = ci.w > 0;
    if (has_in) {
      // S_in rows e, columns n (the columns from DK to the next multiple of 32 stay zero: the
      // keys' padding)
      const int n4s = P.DV * (P.DK / 4);
#pragma unroll
      for (int it = 0; it < kMaxDV * kMaxDK / 4 / kBlock; ++it) {
        const int e = (int)threadIdx.x + it * kBlock;
        if (e >= n4s) break;
        const int fe = e / (P.DK / 4), n4 = e - fe * (P.DK / 4);
        const float4 v4 = cur.s[it];
        const uint32_t h0 = bf_hi(v4.x), h1 = bf_hi(v4.y), h2 = bf_hi(v4.z), h3 = bf_hi(v4.w);
        *reinterpret_cast<uint2*>(sKS[0] + fe * kLdB + 4 * n4) = make_uint2(h0 | (h1 << 16), h2 | (h3 << 16));
        *reinterpret_cast<uint2*>(sKS[1] + fe * kLdB + 4 * n4) =
            make_uint2(bf_lo(v4.x, h0) | (bf_lo(v4.y, h1) << 16), bf_lo(v4.z, h2) | (bf_lo(v4.w, h3) << 16));
      }
    }
    __syncthreads();
    // the next chunk's row scalars (this chunk's and its entering state are used up), ahead of
    // this chunk's stores
    if (more) {
      issue_order();
      fetch_row_scalars(rf, P, cn, cin, h);
      issue_order();
    }
    if (has_tile) {
      const int ib = tib, eb = teb;
      f32x4 y = {0.f, 0.f, 0.f, 0.f};
      if (has_in) {
        for (int ks = 0; ks < nks; ++ks) {
          const int ao = (ib * 16 + lr) * kLdB + 32 * ks + 8 * lg, bo = (eb * 16 + lr) * kLdB + 32 * ks + 8 * lg;
          y = mfma3(lds16(sQ[0] + ao), lds16(sQ[1] + ao), lds16(sKS[0] + bo), lds16(sKS[1] + bo), y);
        }
#pragma unroll
        for (int r = 0; r < 4; ++r) y[r] *= __expf(L.cs[ib * 16 + 4 * lg + r]);
      }
      // both 32-column steps: M is zero above its diagonal tiles and v past the chunk's end; v
      // is exact in bf16, so M's two halves take one product each
#pragma unroll
      for (int js = 0; js < kC / 32; ++js) {
        const int ao = (ib * 16 + lr) * kLdT + 32 * js + 8 * lg;
        const u32x4 vb = lds16(sVt + (eb * 16 + lr) * kLdT + 32 * js + 8 * lg);
        y = mfma_bf(lds16(sM[0] + ao), vb, y);
        y = mfma_bf(lds16(sM[1] + ao), vb, y);
      }
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int i = ib * 16 + 4 * lg + r;
        if (i < ci.z) {
          const size_t o = ((size_t)(ci.y + i) * P.H + h) * P.DV + f;
          P.out[o] = (bf16_t)f32_to_bf16(y[r] * zf[r] * sigmoidf_(zf[r]));
        }
      }
    }
    if (!more) break;
    // the next chunk's gate inputs, ahead of the prefetch after it
    issue_order();
    fetch_gate(zf, cin);
    __syncthreads();  // every wave is done with this chunk's LDS
    c = cn;
    ci = cin;
    si = sil;
    cur = nxt;
    cn = cnn;
    cin = cinn;
  }
}

size_t al256(size_t v) { return (v + 255) & ~(size_t)255; }

// The operator's arguments (device pointers unless noted).
struct M3Args {
  void* out;
  void* fin_angle;
  float* fin_ssm;
  float* fin_k;
  void* fin_v;
  const void *q, *k, *v;
  const float *adt, *dt;
  const void* trap;
  const float *q_bias, *k_bias;
  const void* angles;
  const float* d;
  const void* z;
  const int32_t* cu_seqlens;
  int32_t num_seqs;
  int64_t num_rows;
  mamba3_dims dims;
};

}  // namespace

// Workspace layout of the Mamba-3 forward (each section 256-byte aligned).
struct M3Layout {
  int64_t nch;
  size_t off_seq, off_chunk, off_ang, off_dec, off_state, total;
};

M3Layout m3_layout(const mamba3_varlen* b, const mamba3_dims* d) {
  M3Layout L{};
  int64_t nch = 0;
  for (int s = 0; s < b->num_seqs; ++s) nch += (b->run_lengths[s] + kC - 1) / kC;
  L.nch = nch;
  size_t off = 0;
  L.off_seq = off;
  off = al256(off + (size_t)b->num_seqs * sizeof(int2));
  L.off_chunk = off;
  off = al256(off + (size_t)nch * sizeof(int4));
  L.off_ang = off;
  off = al256(off + (size_t)nch * d->nheads * d->nangles * sizeof(float));
  L.off_dec = off;
  off = al256(off + (size_t)nch * d->nheads * sizeof(float));
  L.off_state = off;
  off = al256(off + (size_t)nch * d->nheads * d->v_dim * d->qk_dim * sizeof(float));
  L.total = off;
  return L;
}

bool m3_supported(const mamba3_dims* d) {
  // the matrix tiles are 16 wide in both widths
  return d->nheads >= 1 && d->qk_dim >= 16 && d->qk_dim <= kMaxDK && d->qk_dim % 16 == 0 && d->v_dim >= 16 &&
         d->v_dim <= kMaxDV && d->v_dim % 16 == 0 && d->nangles >= 0 && d->nangles <= kMaxNA &&
         2 * d->nangles <= d->qk_dim;
}

hipError_t launch_segment_tables(const int32_t* cu, int S, int seg_len, int2* seq_info, int4* seg_info,
                                 hipStream_t st);

namespace {
hipError_t launch_mamba3_forward(const M3Args& a, const M3Layout& lay, char* ws, hipStream_t st) {
  M3Ptrs P{};
  P.q = (const bf16_t*)a.q;
  P.k = (const bf16_t*)a.k;
  P.v = (const bf16_t*)a.v;
  P.adt = a.adt;
  P.dt = a.dt;
  P.trap = (const bf16_t*)a.trap;
  P.q_bias = a.q_bias;
  P.k_bias = a.k_bias;
  P.angles = (const bf16_t*)a.angles;
  P.d = a.d;
  P.z = (const bf16_t*)a.z;
  P.out = (bf16_t*)a.out;
  P.fin_angle = (bf16_t*)a.fin_angle;
  P.fin_ssm = a.fin_ssm;
  P.fin_k = a.fin_k;
  P.fin_v = (bf16_t*)a.fin_v;
  P.seq_info = (const int2*)(ws + lay.off_seq);
  P.chunk_info = (const int4*)(ws + lay.off_chunk);
  P.ang_tot = (float*)(ws + lay.off_ang);
  P.decay = (float*)(ws + lay.off_dec);
  P.state = (float*)(ws + lay.off_state);
  P.H = a.dims.nheads;
  P.DK = a.dims.qk_dim;
  P.DV = a.dims.v_dim;
  P.NA = a.dims.nangles;
  P.T = (int)a.num_rows;
  const int S = a.num_seqs;
  const int nch = (int)lay.nch;
  int2* seq_out = (int2*)(ws + lay.off_seq);
  int4* chunk_out = (int4*)(ws + lay.off_chunk);
  const bool own_tables = P.NA > 0 && S <= kTableSeqs;  // the angle-totals launch builds them
  if (!own_tables) {
    hipError_t e = launch_segment_tables(a.cu_seqlens, S, kC, seq_out, chunk_out, st);
    if (e != hipSuccess) return e;
  }
  if (P.NA > 0) {
    const dim3 ag((unsigned)nch, (unsigned)((P.H + kAngHeads - 1) / kAngHeads));
    if (own_tables) {
      M2_LAUNCH("m3_angle_totals", m3_angle_totals_kernel<true>, ag, dim3(256), 0, st, P, nch, a.cu_seqlens, S,
                seq_out, chunk_out);
    } else {
      M2_LAUNCH("m3_angle_totals", m3_angle_totals_kernel<false>, ag, dim3(256), 0, st, P, nch, a.cu_seqlens, S,
                seq_out, chunk_out);
    }
    M2_LAUNCH("m3_angle_prefix", m3_angle_prefix_kernel, dim3((unsigned)S, (unsigned)((P.H * P.NA + 255) / 256)),
              dim3(256), 0, st, P, S);
  }
  const bool fixed = P.DK == 128 && P.DV == 64 && P.NA <= 32;  // the workloads' shape
  if (fixed) {
    M2_LAUNCH("m3_chunk_state", (m3_chunk_state_kernel<128, 64, 32>), dim3((unsigned)nch, (unsigned)P.H),
              dim3(kBlock), 0, st, P, nch);
  } else {
    M2_LAUNCH("m3_chunk_state", (m3_chunk_state_kernel<0, 0, kMaxNA>), dim3((unsigned)nch, (unsigned)P.H),
              dim3(kBlock), 0, st, P, nch);
  }
  const int f4 = P.DV * P.DK / 4;
  M2_LAUNCH("m3_pass", m3_pass_kernel, dim3((unsigned)((f4 + 255) / 256), (unsigned)P.H, (unsigned)(S < 65535 ? S : 65535)),
            dim3(256), 0, st, P, S);
  // output workgroups: one per CU (their LDS) over the 256 CUs, each taking every ngrp-th chunk
  // of its head
  const int ngrp = (int)std::min<int64_t>(nch, std::max<int64_t>(1, (256 + P.H - 1) / P.H));
  if (fixed) {
    M2_LAUNCH("m3_chunk_out", (m3_chunk_out_kernel<128, 64, 32>), dim3((unsigned)ngrp, (unsigned)P.H),
              dim3(kBlock), 0, st, P, nch);
  } else {
    M2_LAUNCH("m3_chunk_out", (m3_chunk_out_kernel<0, 0, kMaxNA>), dim3((unsigned)ngrp, (unsigned)P.H),
              dim3(kBlock), 0, st, P, nch);
  }
  return hipSuccess;
}

bool aligned16_all(std::initializer_list<const void*> ps) {
  for (const void* p : ps)
    if (((uintptr_t)p & 15) != 0) return false;
  return true;
}

// Run lengths: each >= 1, summing to num_rows; sizes within 32-bit element offsets.
mamba2_status m3_check(const mamba3_varlen* b, const mamba3_dims* d) {
  if (!b || !d) return MAMBA2_INVALID_ARGUMENT;
  if (b->num_seqs < 0 || b->num_rows < 0) return MAMBA2_INVALID_ARGUMENT;
  if (d->nheads < 1 || d->qk_dim < 1 || d->v_dim < 1 || d->nangles < 0 || 2 * (int64_t)d->nangles > d->qk_dim)
    return MAMBA2_INVALID_ARGUMENT;
  if (b->num_seqs > 0 && (!b->run_lengths || !b->dev_cu_seqlens)) return MAMBA2_INVALID_ARGUMENT;
  int64_t sum = 0;
  for (int s = 0; s < b->num_seqs; ++s) {
    if (b->run_lengths[s] < 1) return MAMBA2_RUN_LENGTHS;
    sum += b->run_lengths[s];
  }
  if (sum != b->num_rows) return MAMBA2_RUN_LENGTHS;
  if (!m3_supported(d)) return MAMBA2_NOT_IMPLEMENTED;
  const int64_t T = b->num_rows;
  if (T * d->nheads * d->v_dim >= ((int64_t)1 << 31) || T * d->qk_dim >= ((int64_t)1 << 31))
    return MAMBA2_NOT_IMPLEMENTED;
  return MAMBA2_OK;
}
}  // namespace

}  // namespace m2

using namespace m2;

extern "C" {

size_t mamba3_siso_forward_workspace_bytes(const mamba3_varlen* batch, const mamba3_dims* dims) {
  if (m3_check(batch, dims) != MAMBA2_OK || batch->num_rows == 0) return 0;
  return m3_layout(batch, dims).total;
}

mamba2_status mamba3_siso_forward(void* out, void* final_angle, float* final_ssm, float* final_k, void* final_v,
                                  const void* q, const void* k, const void* v, const float* adt, const float* dt,
                                  const void* trap, const float* q_bias, const float* k_bias, const void* angles,
                                  const float* d, const void* z, const mamba3_varlen* batch, const mamba3_dims* dims,
                                  void* workspace, size_t workspace_bytes, void* stream) {
  mamba2_status st = m3_check(batch, dims);
  if (st != MAMBA2_OK) return st;
  if (batch->num_rows == 0) return MAMBA2_OK;
  if (!out || (dims->nangles > 0 && !final_angle) || !final_ssm || !final_k || !final_v || !q || !k || !v || !adt ||
      !dt || !trap || !q_bias || !k_bias || (dims->nangles > 0 && !angles) || !d || !z)
    return MAMBA2_INVALID_ARGUMENT;
  if (!aligned16_all({out, final_ssm, final_k, q, k, v, z, q_bias, k_bias})) return MAMBA2_INVALID_ARGUMENT;
  const M3Layout lay = m3_layout(batch, dims);
  if (!workspace || workspace_bytes < lay.total) return MAMBA2_WORKSPACE_TOO_SMALL;
  if (((uintptr_t)workspace & 255) != 0) return MAMBA2_INVALID_ARGUMENT;
  M3Args a{out, final_angle, final_ssm, final_k, final_v, q, k, v, adt, dt, trap, q_bias, k_bias, angles, d, z,
           batch->dev_cu_seqlens, batch->num_seqs, batch->num_rows, *dims};
  return launch_mamba3_forward(a, lay, (char*)workspace, (hipStream_t)stream) == hipSuccess ? MAMBA2_OK
                                                                                            : MAMBA2_HIP_ERROR;
}

}  // extern "C"
