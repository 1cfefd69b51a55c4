// Chunked selective scan on MFMA for gfx950: bf16 activations, headdim 64, d_state 128.
//
// The recurrence ("feat(backend): Mamba2 ops, with CPU reference implementations",
// section "Ops", SSMScan) summed in closed form over chunks of 64 rows ("Granite Mamba2
// Inference Optimization": long prefill as a chunked parallel scan).  Per chunk and head,
// with a_t = -exp(A_log) dt'_t, cs_i = sum_{t<=i} a_t inside the chunk, G = C B^T and S
// the state entering the chunk:
//   y_i  = exp(cs_i) C_i . S + sum_{j<=i} G_ij exp(cs_i - cs_j) dt'_j x_j + D x_i
//   S'   = exp(cs_63) S + sum_j exp(cs_63 - cs_j) dt'_j x_j (x) B_j
//
// The state is carried in a frame, S = lam * Sh: the chunk decay then folds into per-row
// weights (y's row scale exp(cs_i) lam, the update weights exp(cs_63 - cs_j) dt'_j / lam'),
// and Sh is only rescaled when lam' = lam exp(cs_63) drops below 2^-20 (Sh <- lam' Sh,
// lam' <- 1), or restarted from zero when the chunk decays by more than e^-60 (the carried
// state's share is then below fp32 resolution).  Intra-chunk weights exp(cs_i - cs_j) are
// per element on the diagonal 16 x 16 blocks and exp(cs_i - cs_b) exp(cs_b - cs_j), b the
// last row of j's block (both factors at most 1), off the diagonal.
//
// Contractions run on v_mfma_f32_16x16x32_bf16 (fp32 accumulate).  x, B and C are exact in
// bf16; M, Sh and w o x are fp32 values split into bf16 hi + lo halves (two MFMAs each): y
// sums terms that cancel and the fp32 state needs ~16 bits per step.
//
// Mapping.  A workgroup walks one segment (a run of chunks of one sequence) for HB heads of
// one group with 2 HB waves; wave (head hh, half ph) owns state rows p in [32 ph, 32 ph + 32)
// of its head (all n) and the matching 32 columns of y.  The state lives in MFMA accumulators
// as S^T tiles (n x p) whose lane layout is the A-operand layout of S C^T, so the state never
// goes through LDS.  G^T = B C^T is computed once per chunk for all HB heads (its first eight
// 16 x 16 tiles dealt over the waves, the last two per head by that head's waves), scaled per
// head into M^T and shared through LDS in operand order.  Chunk rows of B, C and x are copied
// global -> LDS by buffer loads that write LDS directly, XOR-swizzled in 16-byte units, into
// single tiles: the next chunk's copies are issued once the current tiles are no longer read
// and land during the output phase, while the CU's other workgroup computes.  The transposed
// operands (x^T, B^T) come from the gfx950 transposing LDS read.  Contractions
// use permuted k orders that match the accumulator layout (lane group g holds rows 4 g..4 g+3
// of a 16 x 16 tile): over chunk rows j, slot s of group g in k block m is
// j = 32 m + 16 (s / 4) + 4 g + s % 4 (two stacked tiles).  State tile nb holds the columns
// n = 32 (nb / 2) + 8 (R / 4) + 4 (nb % 2) + R % 4 in its rows R (the transposing reads of B
// pick them), so that in S C^T block kk pairs tiles 2 kk and 2 kk + 1 and slot s of group g is
// n = 32 kk + 8 g + s: a lane's C operand is one 16-byte read.
#include "common.h"

#include <type_traits>

namespace m2 {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef short i16x4 __attribute__((ext_vector_type(4)));

#define M2_LDS __attribute__((address_space(3)))

constexpr int kP = 64;   // head dim
constexpr int kN = 128;  // state dim
constexpr int kQ = 64;   // chunk rows
constexpr float kFrameMin = 0x1p-20f;  // smallest state-frame scale before a rescale
constexpr float kDropSpan = 60.f;      // a chunk decaying by more than e^-60 drops the carried state
constexpr int kTiles = 10;             // lower-triangular 16 x 16 tiles of a 64 x 64 chunk
constexpr int kMaxSegChunks = 64;      // chunks per segment at most (segments of <= 4096 rows)

// Per-chunk decay quantities of one head (written by the head's two waves, read by all).
struct Decay {
  float e[kQ];      // exp(cs_i) lam
  float dt[kQ];     // dt'_j
  float cs[kQ];     // cs_i
  float w[kQ];      // exp(cs_63 - cs_j) dt'_j / lam'
  float ef[kQ];     // exp(cs_b - cs_j) dt'_j, b the last row of j's 16-row block
  float er[3][kQ];  // exp(cs_i - cs_b), b = 16 jb + 15, for rows i past block jb
  float scale;      // state factor before this chunk's update: 1 keep, 0 drop, else rescale
  float lam_next;   // lam'
  float pad[2];
};

struct SegPtrs {
  const int2* seq_info;
  const int4* seg_info;
  float* seg_decay;
  float* seg_state;
  int* seg_start;    // [nseg][H]: first chunk the local-state walk takes | kTailLeft when skipped
  float* seg_chunk;  // [nseg][kMaxSegChunks][H]: log-decay sums of the segment's chunks
  int tail_ok;       // the output kernel may compute a dropped predecessor's state itself
};

// seg_start flag: the segment-state kernel left this segment's local state to the output
// kernel of the next segment (its index in seg_state is not written).
constexpr int kTailLeft = 1 << 8;

// ------------------------------------------------------------------ small helpers

__device__ __forceinline__ f32x4 mfma(const u32x4& a, const u32x4& b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a), __builtin_bit_cast(bf16x8, b),
                                                  c, 0, 0, 0);
}
__device__ __forceinline__ uint32_t pk(float lo, float hi) {
  bf16x2 v = {(__bf16)lo, (__bf16)hi};
  return __builtin_bit_cast(uint32_t, v);
}
__device__ __forceinline__ float lo_f(uint32_t u) { return __uint_as_float(u << 16); }
__device__ __forceinline__ float hi_f(uint32_t u) { return __uint_as_float(u & 0xffff0000u); }
__device__ __forceinline__ int uniform(int v) { return __builtin_amdgcn_readfirstlane(v); }
// The same value, hidden from the optimiser: addresses derived from it are recomputed where
// used instead of being kept live across the chunk loop.
__device__ __forceinline__ int opaque(int v) {
  asm volatile("" : "+v"(v));
  return v;
}
__device__ __forceinline__ float uniformf(float v) {
  return __int_as_float(__builtin_amdgcn_readfirstlane(__float_as_int(v)));
}

// Split 4 fp32 values into packed bf16 hi (x, y) and lo (z, w) halves.
// The packed hi halves pass through an empty asm so that the lo halves are formed from
// them (one shift or mask each) instead of from a second conversion.
__device__ __forceinline__ uint32_t pk_hi(float lo, float hi) {
  uint32_t h = pk(lo, hi);
  asm("" : "+v"(h));
  return h;
}
__device__ __forceinline__ u32x4 split4(float v0, float v1, float v2, float v3) {
  const uint32_t h01 = pk_hi(v0, v1), h23 = pk_hi(v2, v3);
  return u32x4{h01, h23, pk(v0 - lo_f(h01), v1 - hi_f(h01)), pk(v2 - lo_f(h23), v3 - hi_f(h23))};
}

typedef __amdgpu_buffer_rsrc_t Rsrc;
// Buffer resource over `bytes` bytes from `base`: lane offsets (voffset) at or past the end
// read as zero and drop writes.  The uniform soffset adds to the address, not to the range.
__device__ __forceinline__ Rsrc make_rsrc(const void* base, int64_t bytes) {
  const int n = bytes <= 0 ? 0 : (int)bytes;
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, n, 0x00020000);
}
// bf16 bits of dt[r0 + lane][h] for lanes below nr, else 0: a branch-free load whose value
// is only waited for where it is converted.
__device__ __forceinline__ uint32_t dt_bits(const bf16_t* dt, int r0, int nr, int H, int h, int lane) {
  const Rsrc r = make_rsrc(dt + (size_t)r0 * H + h, (int64_t)nr * H * 2);
  return __builtin_amdgcn_raw_buffer_load_b16(r, (uint32_t)(lane * H * 2), 0, 0);
}
__device__ __forceinline__ void bst8(Rsrc r, uint32_t voff, uint32_t soff, u32x2 v) {
  __builtin_amdgcn_raw_buffer_store_b64(v, r, voff, soff, 0);
}
// 16 bytes per lane from global memory into LDS at lds + 16 * lane (lds wave-uniform): a
// buffer load that writes LDS, through a descriptor over `bytes` bytes from `base` (dma_rsrc:
// one per chunk and tile kind; lane offsets voff at or past `bytes` write zeros, the uniform
// soff moves the address without entering the range check).  Issued from inline assembly so
// that the compiler, which cannot tell these LDS writes apart from the tiles being read
// meanwhile, adds no waits of its own; the copies are waited for (vmcnt 0) before the barrier
// that publishes them.
typedef uint32_t u32x4s __attribute__((ext_vector_type(4)));
#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"  // m0 is set here and used by nothing else
__device__ __forceinline__ u32x4s dma_rsrc(const char* base, int bytes) {
  const uint64_t a = (uint64_t)base;
  return u32x4s{(uint32_t)a, (uint32_t)(a >> 32) & 0xffffu, bytes <= 0 ? 0u : (uint32_t)bytes, 0x00020000u};
}
__device__ __forceinline__ void dma16(const u32x4s& rsrc, const bf16_t* lds, uint32_t voff, uint32_t soff) {
  const uint32_t m0 = (uint32_t)(uintptr_t)(const M2_LDS void*)lds;
  asm volatile("s_mov_b32 m0, %0\n\tbuffer_load_dwordx4 %1, %2, %3 offen lds"
               :
               : "s"(m0), "v"(voff), "s"(rsrc), "s"(soff)
               : "m0");
}
#pragma clang diagnostic pop

// XOR swizzles of 16-byte units within tile rows, linear in the bits of row % 16.  B and C
// tiles (256-byte rows, 16 units) use a 4-bit map and x tiles (128-byte rows, 8 units) a
// 3-bit one; both were chosen by timing every such map on the reads below (row reads of 16
// consecutive rows, 8-byte fragment reads, transposing reads of 4-row groups), which then
// run without bank conflicts.  Offsets that cross into the other half of a B / C row flip
// unit bit 3 (element offset bit 6), so they are applied with XOR, not addition.
__device__ __forceinline__ int swz_bc(int row) {
  return ((row & 1) ? 3 : 0) ^ ((row & 2) ? 6 : 0) ^ ((row & 4) ? 8 : 0) ^ ((row & 8) ? 12 : 0);
}
__device__ __forceinline__ int swz_x(int row) {
  return ((row & 1) ? 4 : 0) ^ ((row & 2) ? 5 : 0) ^ ((row & 4) ? 6 : 0) ^ ((row & 8) ? 4 : 0);
}

template <typename T>
__device__ __forceinline__ u32x4 lds16(const T* p) { return *reinterpret_cast<const u32x4*>(p); }

// Transposing read: within each 16-lane group, lane c receives column c of the four rows
// whose 8-byte pieces the group's lanes address (lane l: row (l % 16) / 4, columns 4 (l % 4)).
__device__ __forceinline__ u32x2 tr8(const bf16_t* p) {
  const i16x4 v = __builtin_amdgcn_ds_read_tr16_b64_v4i16((M2_LDS i16x4*)p);
  return __builtin_bit_cast(u32x2, v);
}

// Per-lane element offsets into the swizzled tiles (B and C: [64][128], x: [64][64]).
// Lane (c, g) = (lane % 16, lane / 16); q = (lane % 16) / 4, b = (lane % 4) / 2.
struct Lofs {
  int gt[2];  // B / C row 16 jb + c, elements 32 kk + 8 g..: + 16 jb*128, [kk%2], ^ 64 (kk/2)
  int cf[4];  // C row 16 ib + c, elements 32 kk + 8 g .. +7: + 16 ib*128, [kk]
  int bt;     // B^T transposing read of state tile nb: ^ 32 (nb / 2), + 4 (nb % 2)
  int xt[2];  // x^T transposing read for p block 32 ph + 16 t: + row0*64, [t]
};
__device__ __forceinline__ Lofs lane_offsets(int lane, int ph) {
  const int g = lane >> 4, c = lane & 15, q = (lane & 15) >> 2, b = (lane & 3) >> 1, e = 4 * (lane & 1);
  const int sc = swz_bc(c), sq = swz_bc(4 * g + q), sx = swz_x(4 * g + q);
  Lofs o;
#pragma unroll
  for (int a = 0; a < 2; ++a) o.gt[a] = c * kN + (((4 * a + g) ^ sc) << 3);
#pragma unroll
  for (int kk = 0; kk < 4; ++kk) o.cf[kk] = c * kN + (((4 * kk + g) ^ sc) << 3);
  o.bt = (4 * g + q) * kN + (((lane & 3) ^ sq) << 3);
#pragma unroll
  for (int t = 0; t < 2; ++t) o.xt[t] = (4 * g + q) * kP + (((4 * ph + 2 * t + b) ^ sx) << 3) + e;
  return o;
}

// Operand whose lane (c, g) holds T[j][col c] for the 8 k slots j of block m (T row-major,
// k = row index); `base` is the tile plus the lane's transposing-read offset.
template <int W>
__device__ __forceinline__ u32x4 tr_frag(const bf16_t* base, int m) {
  const u32x2 a = tr8(base + 32 * m * W);
  const u32x2 b = tr8(base + (32 * m + 16) * W);
  return u32x4{a.x, a.y, b.x, b.y};
}

// x + (x from another lane by the DPP control `ctrl`, 0 where there is none), on the rows
// in row_mask.  All 64 lanes must be active.
template <int kCtrl, int kRowMask>
__device__ __forceinline__ float dpp_add(float x) {
  return x + __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), kCtrl, kRowMask, 0xf, false));
}
// Inclusive prefix sum over the 64 lanes: shifts within 16-lane rows, then the row totals
// broadcast forward (lane 15 to row 1 and 3, lane 31 to rows 2 and 3).
__device__ __forceinline__ float wave_scan_incl(float v) {
  v = dpp_add<0x111, 0xf>(v);  // row_shr:1
  v = dpp_add<0x112, 0xf>(v);  // row_shr:2
  v = dpp_add<0x114, 0xf>(v);  // row_shr:4
  v = dpp_add<0x118, 0xf>(v);  // row_shr:8
  v = dpp_add<0x142, 0xa>(v);  // row_bcast:15
  v = dpp_add<0x143, 0xc>(v);  // row_bcast:31
  return v;
}
__device__ __forceinline__ float lane_value(float v, int l) {
  return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), l));
}

// M^T operand (ib, m), m <= ib / 2, holds tiles jb = 2 m (slots 0..3) and 2 m + 1 (slots
// 4..7) of column block ib.  LDS keeps it in 1 KB units of [64 lanes][16 bytes]: two units
// (hi, lo) for a full operand; one unit {hi of jb, lo of jb} when tile 2 m + 1 lies above
// the diagonal (operands (0, 0) and (2, 1)).
__device__ __forceinline__ constexpr int m_unit(int ib, int m) {
  return ib == 0 ? 0 : ib == 1 ? 1 : ib == 2 ? (m == 0 ? 3 : 5) : (m == 0 ? 6 : 8);
}
__device__ __forceinline__ constexpr bool m_half(int ib, int m) { return (ib == 0) || (ib == 2 && m == 1); }

// Workgroup b runs on XCD b % 8; give each XCD a contiguous range of work items so the
// head groups of one segment share that XCD's L2.
__device__ __forceinline__ int work_item(int b, int n) {
  const int x = b & 7;
  return x * (n >> 3) + min(x, n & 7) + (b >> 3);
}

// ------------------------------------------------------------------ per-chunk pieces

// Decay quantities of one head for a chunk (lane = chunk row, v = raw dt).  Both waves of
// the head compute dt' and the prefix sums; half 0 writes the row scales and the diagonal
// weights, half 1 the update and off-diagonal weights and the scalars.  lam is the frame
// scale entering the chunk; it and lsum (sum of chunk log-decays) advance in both waves.
__device__ __forceinline__ void chunk_decay(Decay& d, float v, float A, float bias, int nr, int lane, int ph,
                                            float& lam, float& lsum) {
  const float dtp = lane < nr ? softplus_f32(v + bias) : 0.f;
  const float cs = wave_scan_incl(-A * dtp);
  const float cend = lane_value(cs, 63);
  const float tent = lam * __expf(cend);
  const bool reset = tent < kFrameMin;
  const float lam_next = reset ? 1.f : tent;
  const float b0 = lane_value(cs, 15), b1 = lane_value(cs, 31), b2 = lane_value(cs, 47);
  if (ph == 0) {
    d.e[lane] = __expf(cs) * lam;
    d.dt[lane] = dtp;
    d.cs[lane] = cs;
    d.er[0][lane] = __expf(cs - b0);
    d.er[1][lane] = __expf(cs - b1);
    d.er[2][lane] = __expf(cs - b2);
  } else {
    d.w[lane] = __expf(cend - cs) * dtp * __builtin_amdgcn_rcpf(lam_next);
    const int r = lane >> 4;
    const float cb = r == 0 ? b0 : r == 1 ? b1 : r == 2 ? b2 : cend;
    d.ef[lane] = __expf(cb - cs) * dtp;
    if (lane == 0) {
      d.scale = -cend > kDropSpan ? 0.f : (reset ? tent : 1.f);
      d.lam_next = lam_next;
    }
  }
  lam = lam_next;
  lsum += cend;
}

// The segment-state pass needs only the update weights and the frame scalars: both waves
// of the head compute them, half 1 writes them.
__device__ __forceinline__ void chunk_decay_update(Decay& d, float v, float A, float bias, int nr, int lane, int ph,
                                                   float& lam, float& lsum) {
  const float dtp = lane < nr ? softplus_f32(v + bias) : 0.f;
  const float cs = wave_scan_incl(-A * dtp);
  const float cend = lane_value(cs, 63);
  const float tent = lam * __expf(cend);
  const bool reset = tent < kFrameMin;
  const float lam_next = reset ? 1.f : tent;
  if (ph == 1) {
    d.w[lane] = __expf(cend - cs) * dtp * __builtin_amdgcn_rcpf(lam_next);
    if (lane == 0) {
      d.scale = -cend > kDropSpan ? 0.f : (reset ? tent : 1.f);
      d.lam_next = lam_next;
    }
  }
  lam = lam_next;
  lsum += cend;
}

// A wave's B / C copy instructions all have block index k = w (mod 4) and its x copies
// k = w (mod 2) (see load_bc, load_x), so one lane offset per wave serves each kind.
struct DmaOfs {
  uint32_t bc;  // B / C block rows
  uint32_t x;   // x block rows
};
__device__ __forceinline__ DmaOfs dma_offsets(int lane, int w, uint32_t ld) {
  DmaOfs o;
  const int r = lane >> 4;  // row 4 k + r of the tile, unit lane % 16
  o.bc = 2u * ((uint32_t)r * ld + 8u * (uint32_t)((lane & 15) ^ swz_bc(4 * (w & 3) + r)));
  const int rx = lane >> 3;  // row 8 k + rx, unit lane % 8
  o.x = 2u * ((uint32_t)rx * ld + 8u * (uint32_t)((lane & 7) ^ swz_x(8 * (w & 1) + rx)));
  return o;
}

// Global -> LDS copies of chunk rows [r0, r0 + nr): each instruction fills 1 KB of a tile
// (4 rows of a [64][128] B or C tile, 8 rows of a [64][64] x tile), each lane fetching the
// global 16-byte unit that the swizzle places at its LDS slot; rows past nr read as zero.
// Instructions are dealt round robin to the 2 HB waves.
// rows: the chunk's first row; nrb: its valid bytes (rows x row pitch); ldb: row pitch in bytes
template <int HB, int NT>
__device__ __forceinline__ void load_bc(const bf16_t* rows, int nrb, uint32_t ldb, const uint32_t (&col)[NT],
                                        bf16_t* const (&dst)[NT], const DmaOfs& o, int w) {
  constexpr int nW = 2 * HB;
  static_assert(16 % nW == 0, "instruction split");
  const u32x4s rs = dma_rsrc(reinterpret_cast<const char*>(rows), nrb);
#pragma unroll
  for (int i = 0; i < 16 * NT / nW; ++i) {
    const int tile = nW * i / 16;  // compile time
    const int k = (w + nW * i) & 15;
    dma16(rs, dst[tile] + 512 * k, o.bc + (uint32_t)(4 * k) * ldb, 2u * col[tile]);  // k % 4 == w % 4
  }
}
template <int HB>
__device__ __forceinline__ void load_x(const bf16_t* rows, int nrb, uint32_t ldb, uint32_t colX,
                                       bf16_t (*sX)[kQ * kP], const DmaOfs& o, int w) {
  constexpr int nW = 2 * HB;
  const u32x4s rs = dma_rsrc(reinterpret_cast<const char*>(rows), nrb);
#pragma unroll
  for (int i = 0; i < 8 * HB / nW; ++i) {
    const int t = w + nW * i;
    const int hh = t >> 3, k = t & 7;
    dma16(rs, sX[hh] + 512 * k, o.x + (uint32_t)(8 * k) * ldb, 2u * (colX + (uint32_t)(hh * kP)));
  }
}

// w o x operands (hi, lo) of k block m from the x^T operand of the same block.
__device__ __forceinline__ void wx_frag(const u32x4& xt, const Decay& d, int m, int lane, u32x4& hi, u32x4& lo) {
  const int g = lane >> 4;
  const f32x4 w0 = *reinterpret_cast<const f32x4*>(&d.w[32 * m + 4 * g]);
  const f32x4 w1 = *reinterpret_cast<const f32x4*>(&d.w[32 * m + 16 + 4 * g]);
  const u32x4 a = split4(w0[0] * lo_f(xt[0]), w0[1] * hi_f(xt[0]), w0[2] * lo_f(xt[1]), w0[3] * hi_f(xt[1]));
  const u32x4 b = split4(w1[0] * lo_f(xt[2]), w1[1] * hi_f(xt[2]), w1[2] * lo_f(xt[3]), w1[3] * hi_f(xt[3]));
  hi = u32x4{a[0], a[1], b[0], b[1]};
  lo = u32x4{a[2], a[3], b[2], b[3]};
}

// S^T(nb, pb) (+)= B^T (w o x) for the wave's two p blocks; kFresh starts from zero.
template <bool kFresh>
__device__ __forceinline__ void su_mfma(f32x4 (&S)[2][8], const u32x4 (&wh)[2][2], const u32x4 (&wl)[2][2],
                                        const bf16_t* sB, const Lofs& lo) {
#pragma unroll
  for (int nb = 0; nb < 8; ++nb) {
#pragma unroll
    for (int m = 0; m < 2; ++m) {
      const u32x4 bt = tr_frag<kN>(sB + ((lo.bt ^ (32 * (nb >> 1))) + 4 * (nb & 1)), m);
#pragma unroll
      for (int t = 0; t < 2; ++t) {
        S[t][nb] = mfma(bt, wh[t][m], (kFresh && m == 0) ? f32x4{0.f, 0.f, 0.f, 0.f} : S[t][nb]);
        S[t][nb] = mfma(bt, wl[t][m], S[t][nb]);
      }
    }
  }
}

// State update for the chunk: S <- scale S + B^T (w o x); xt[t][m] are the x^T operands.
__device__ __forceinline__ void state_update(f32x4 (&S)[2][8], const u32x4 (&xt)[2][2], const bf16_t* sB,
                                             const Lofs& lo, const Decay& d, int lane) {
  u32x4 wh[2][2], wl[2][2];
#pragma unroll
  for (int t = 0; t < 2; ++t)
#pragma unroll
    for (int m = 0; m < 2; ++m) wx_frag(xt[t][m], d, m, lane, wh[t][m], wl[t][m]);
  const float scale = uniformf(d.scale);
  if (scale == 0.f) {
    su_mfma<true>(S, wh, wl, sB, lo);
  } else {
    if (scale != 1.f) {
#pragma unroll
      for (int t = 0; t < 2; ++t)
#pragma unroll
        for (int nb = 0; nb < 8; ++nb) S[t][nb] *= scale;
    }
    su_mfma<false>(S, wh, wl, sB, lo);
  }
}

// State tile (nb, t) of wave half ph: S[p][n..n+3], p = 32 ph + 16 t + c,
// n = 32 (nb / 2) + 8 g + 4 (nb % 2).
__device__ __forceinline__ size_t state_elem(int ph, int t, int nb, int lane) {
  const int g = lane >> 4, c = lane & 15;
  return (size_t)(32 * ph + 16 * t + c) * kN + 32 * (nb >> 1) + 8 * g + 4 * (nb & 1);
}

// ---------------------------------------------------------------- segment states

// Local state of the segment rows [r0, r0 + nrows) of heads h0.. (two waves per head, B
// and x copied through sB and sX, decays through sD), walked from chunk q0 with a zero
// entering state: on return S holds the wave's rows of S_loc, frame-corrected, and the
// tiles and decay slots are free again.
__device__ __forceinline__ void walk_local_state(f32x4 (&S)[2][8], const bf16_t* xbc, const bf16_t* dt, int r0,
                                                 int nrows, int q0, int H, int h, float A, float bias,
                                                 uint32_t ld, uint32_t colB, uint32_t colX, bf16_t* sB,
                                                 bf16_t (*sX)[kQ * kP], Decay (*sD)[2], const Lofs& lo,
                                                 const DmaOfs& dof, int w, int lane, int hh, int ph) {
  constexpr int HB = 2;
  const int nchunks = (nrows + kQ - 1) / kQ;
  const uint32_t col[1] = {colB};
  auto rows_of = [&](int q) { return xbc + (size_t)(r0 + q * kQ) * ld; };
  auto nr_of = [&](int q) { return min(kQ, nrows - q * kQ); };
  auto dt_of = [&](int q) { return dt_bits(dt, r0 + q * kQ, nr_of(q), H, h, lane); };
  auto load = [&](int q) {
    bf16_t* const dst[1] = {sB};
    const int nrb = nr_of(q) * (int)ld * 2;
    load_bc<HB, 1>(rows_of(q), nrb, 2u * ld, col, dst, dof, w);
    load_x<HB>(rows_of(q), nrb, 2u * ld, colX, sX, dof, w);
  };

#pragma unroll
  for (int t = 0; t < 2; ++t)
#pragma unroll
    for (int nb = 0; nb < 8; ++nb) S[t][nb] = f32x4{0.f, 0.f, 0.f, 0.f};

  float lam = 1.f, lsum = 0.f;
  load(q0);
  chunk_decay_update(sD[q0 & 1][hh], bf16_to_f32(dt_of(q0)), A, bias, nr_of(q0), lane, ph, lam, lsum);
  uint32_t dtn = q0 + 1 < nchunks ? dt_of(q0 + 1) : 0u;

  for (int q = q0; q < nchunks; ++q) {
    const int st = q & 1;
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();  // chunk q rows and decay visible
    u32x4 xt[2][2];
#pragma unroll
    for (int t = 0; t < 2; ++t)
#pragma unroll
      for (int m = 0; m < 2; ++m) xt[t][m] = tr_frag<kP>(sX[hh] + lo.xt[t], m);
    __builtin_amdgcn_s_setprio(1);
    state_update(S, xt, sB, lo, sD[st][hh], lane);
    __builtin_amdgcn_s_setprio(0);
    __syncthreads();  // the tiles are free for the next chunk's copies
    uint32_t dtn2 = 0;
    if (q + 1 < nchunks) {
      load(q + 1);
      if (q + 2 < nchunks) dtn2 = dt_of(q + 2);
    }
    if (q + 1 < nchunks)
      chunk_decay_update(sD[st ^ 1][hh], bf16_to_f32(dtn), A, bias, nr_of(q + 1), lane, ph, lam, lsum);
    dtn = dtn2;
  }
  const float lam_end = uniformf(sD[(nchunks - 1) & 1][hh].lam_next);
#pragma unroll
  for (int t = 0; t < 2; ++t)
#pragma unroll
    for (int nb = 0; nb < 8; ++nb) S[t][nb] *= lam_end;
  __syncthreads();  // every wave has read its frame scale: the decay slots are free
}

// Log-decay sums of every chunk of every segment, per head (those of a sequence's last segment
// are not used; computing them spares a dependent load of the sequence table): the sum of
// a_t = -exp(A_log) softplus(dt_t + dt_bias) over the chunk's rows.  One workgroup per (segment,
// chunk): wave w sums rows [16 w, 16 w + 16) with lane = head (heads in blocks of 64), so that
// each load of dt is one contiguous row and each wave's chain of loads and softplus is a
// quarter of the chunk; wave 0 adds the four partial sums in row order.
constexpr int kSumRows = kQ / 4;

template <bool kTables>
__global__ __launch_bounds__(256) void chunk_sums_kernel(const bf16_t* __restrict__ dt,
                                                         const float* __restrict__ a_log,
                                                         const float* __restrict__ dt_bias, SegPtrs sp, int H,
                                                         int cpb, const int32_t* __restrict__ cu, int S,
                                                         int seg_len, int2* __restrict__ seq_out,
                                                         int4* __restrict__ seg_out) {
  __shared__ float part[4][64];
  const int seg = blockIdx.x / cpb;
  // wave-uniform (the buffer descriptor built from it must be, or each load becomes a loop)
  const int q = uniform((int)(blockIdx.x % cpb));
  const int w = uniform((int)threadIdx.x >> 6), lane = threadIdx.x & 63;
  const int4 si0 = kTables ? own_segment<256>(cu, S, seg_len, seg, seq_out, seg_out, blockIdx.x == 0) : sp.seg_info[seg];
  const int4 si = make_int4(uniform(si0.x), uniform(si0.y), uniform(si0.z), uniform(si0.w));
  if (q * kQ >= si.z) return;  // uniform over the workgroup; no barrier reached yet
  const int nr = min(kQ, si.z - q * kQ);
  const int r0 = w * kSumRows;
  // rows past the chunk's end read as zero and are not summed; lanes past H are unused
  const Rsrc r = make_rsrc(dt + (size_t)(si.y + q * kQ) * H, (int64_t)nr * H * 2);
  for (int hb = 0; hb < H; hb += 64) {  // same trip count in every wave
    const int h = hb + lane;
    const float A = h < H ? __expf(a_log[h]) : 0.f, bias = h < H ? dt_bias[h] : 0.f;
    uint32_t b[kSumRows];  // every row's load in flight before the first is used
#pragma unroll
    for (int i = 0; i < kSumRows; ++i)
      b[i] = __builtin_amdgcn_raw_buffer_load_b16(r, (uint32_t)(((r0 + i) * H + h) * 2), 0, 0);
    float sum = 0.f;
#pragma unroll
    for (int i = 0; i < kSumRows; ++i)
      if (r0 + i < nr) sum += -A * softplus_f32(bf16_to_f32(b[i]) + bias);
    part[w][lane] = sum;
    __syncthreads();
    if (w == 0 && h < H)
      sp.seg_chunk[((size_t)seg * kMaxSegChunks + q) * H + h] =
          ((part[0][lane] + part[1][lane]) + part[2][lane]) + part[3][lane];
    __syncthreads();  // the partial sums are read before the next block of heads overwrites them
  }
}

// From the chunk sums of segment sg (nrows rows), head hd, lane = chunk: the segment's total
// log-decay and the first chunk its local-state walk must take, the last chunk q >= 1 whose
// rows all decay by more than e^-60 before the segment's end (none of the chunks before it
// can change the end state in fp32).
__device__ __forceinline__ int seg_first_chunk(const SegPtrs& sp, int sg, int nrows, int H, int hd, int lane,
                                               float& total) {
  const int nch = (nrows + kQ - 1) / kQ;
  const float c = lane < nch ? sp.seg_chunk[((size_t)sg * kMaxSegChunks + lane) * H + hd] : 0.f;
  const float incl = wave_scan_incl(c);
  total = lane_value(incl, 63);
  const float E = total - incl + c;  // log-decay from the start of chunk `lane` to the segment's end
  const uint64_t drop = __ballot(lane >= 1 && lane < nch && E < -kDropSpan);
  return drop ? 63 - __builtin_clzll(drop) : 0;
}

// Single-buffered tiles: with two heads per workgroup three workgroups fit a CU (LDS and
// registers), and each one's copies are covered by the other two's work.
//
// The walk starts at the earlier of the two heads' first chunks (seg_first_chunk), so
// where the decay is fast only the segment's last chunk or two are walked.  The segment's
// total log-decay gives its decay factor for the pass (0 below -60).  When both
// heads' factors are 0 for this segment and for the next one (or the next is the
// sequence's last), nothing but the output kernel of the next segment reads this local
// state: the walk is left to that kernel (seg_start flag kTailLeft), which does it itself
// from the same chunk with the same arithmetic instead of reading the state back.
__global__ __launch_bounds__(256, 3) void ssd_state_kernel(const bf16_t* __restrict__ xbc,
                                                          const bf16_t* __restrict__ dt,
                                                          const float* __restrict__ a_log,
                                                          const float* __restrict__ dt_bias,
                                                          SegPtrs sp, int H, int G, int nitems) {
  constexpr int HB = 2;
  __shared__ __attribute__((aligned(16))) bf16_t sB[kQ * kN];
  __shared__ __attribute__((aligned(16))) bf16_t sX[HB][kQ * kP];
  __shared__ __attribute__((aligned(16))) Decay sD[2][HB];
  __shared__ int sStart[HB];
  __shared__ int sDead[HB];  // this segment's and the next one's factors both 0

  const int nhg = H / HB;
  const int item = work_item(blockIdx.x, nitems);
  const int seg = item / nhg, h0 = (item % nhg) * HB;
  const int4 si0 = sp.seg_info[seg];
  const int4 si = make_int4(uniform(si0.x), uniform(si0.y), uniform(si0.z), uniform(si0.w));
  if (si.w == uniform(sp.seq_info[si.x].y) - 1) return;  // a sequence's last segment needs no local state

  const int w = uniform((int)threadIdx.x >> 6), lane = threadIdx.x & 63;
  const int hh = w >> 1, ph = w & 1, h = h0 + hh;
  const int Di = H * kP;
  const uint32_t ld = (uint32_t)(Di + 2 * G * kN);
  const int grp = h0 / (H / G);
  const uint32_t colB[1] = {(uint32_t)(Di + grp * kN)};
  const uint32_t colX = (uint32_t)(h0 * kP);
  const float A = __expf(a_log[h]), bias = dt_bias[h];
  const Lofs lo = lane_offsets(lane, ph);
  const DmaOfs dof = dma_offsets(lane, w, ld);

  // first chunk and decay factor per head; the walk left to the next output kernel?
  {
    float total;
    const int q0h = seg_first_chunk(sp, seg, si.z, H, h, lane, total);
    bool dead = total < -kDropSpan;
    if (sp.tail_ok && dead && si.w + 2 < uniform(sp.seq_info[si.x].y)) {
      const int4 sn = sp.seg_info[seg + 1];
      float tn;
      (void)seg_first_chunk(sp, seg + 1, uniform(sn.z), H, h, lane, tn);
      dead = tn < -kDropSpan;
    }
    if (ph == 0 && lane == 0) {
      sStart[hh] = q0h;
      sDead[hh] = dead;
      sp.seg_decay[(size_t)seg * H + h] = total < -kDropSpan ? 0.f : __expf(total);
    }
  }
  __syncthreads();
  const int q0 = uniform(min(sStart[0], sStart[1]));
  const bool left = sp.tail_ok && sDead[0] && sDead[1];
  if (threadIdx.x < HB) sp.seg_start[(size_t)seg * H + h0 + threadIdx.x] = q0 | (left ? kTailLeft : 0);
  if (left) return;  // uniform over the workgroup

  f32x4 S[2][8];
  walk_local_state(S, xbc, dt, si.y, si.z, q0, H, h, A, bias, ld, colB[0], colX, sB, sX, sD, lo, dof, w, lane, hh,
                   ph);

  // S_loc of this segment, at the index of the next segment of the sequence
  float* out = sp.seg_state + ((size_t)(seg + 1) * H + h) * (size_t)(kP * kN);
  const int lane_st = opaque(lane);
#pragma unroll
  for (int t = 0; t < 2; ++t)
#pragma unroll
    for (int nb = 0; nb < 8; ++nb) *reinterpret_cast<f32x4*>(out + state_elem(ph, t, nb, lane_st)) = S[t][nb];
}

// ---------------------------------------------------------------- outputs

// Per chunk: (1) tiles and decay visible -> phase 1: x^T operands, G^T tiles and M^T of the
// workgroup's heads, Y = S C^T, the state update; (2) M^T visible, tiles free -> copies of
// the next chunk, phase 2: Y += x^T M^T, row scales, store, next chunk's decay.
__global__ __launch_bounds__(256, 2) void ssd_scan_kernel(
    bf16_t* __restrict__ y, const bf16_t* __restrict__ xbc, const bf16_t* __restrict__ dt,
    const float* __restrict__ a_log, const float* __restrict__ dt_bias, const float* __restrict__ Dp,
    float* __restrict__ pool, const int32_t* __restrict__ slots, const uint8_t* __restrict__ fresh, SegPtrs sp,
    int H, int G, int nitems, const int32_t* __restrict__ cu, float* __restrict__ snaps, int snapE) {
  constexpr int HB = 2;
  __shared__ __attribute__((aligned(16))) bf16_t sB[kQ * kN];
  __shared__ __attribute__((aligned(16))) bf16_t sC[kQ * kN];
  __shared__ int sRed[4];
  __shared__ __attribute__((aligned(16))) bf16_t sX[HB][kQ * kP];
  __shared__ __attribute__((aligned(16))) u32x4 sM[HB][kTiles][64];
  __shared__ __attribute__((aligned(16))) Decay sD[2][HB];

  const int nhg = H / HB;
  const int item = work_item(blockIdx.x, nitems);
  const int seg = item / nhg, h0 = (item % nhg) * HB;
  const int4 si0 = sp.seg_info[seg];
  const int4 si = make_int4(uniform(si0.x), uniform(si0.y), uniform(si0.z), uniform(si0.w));
  const bool last = si.w == uniform(sp.seq_info[si.x].y) - 1;

  const int w = uniform((int)threadIdx.x >> 6), lane = threadIdx.x & 63;
  const int g = lane >> 4, c = lane & 15;
  const int hh = w >> 1, ph = w & 1, h = h0 + hh;
  const int Di = H * kP;
  const uint32_t ld = (uint32_t)(Di + 2 * G * kN);
  const int grp = h0 / (H / G);
  const uint32_t colBC[2] = {(uint32_t)(Di + grp * kN), (uint32_t)(Di + (G + grp) * kN)};
  const uint32_t colX = (uint32_t)(h0 * kP);
  const float A = __expf(a_log[h]), bias = dt_bias[h];
  float Dh[HB];
#pragma unroll
  for (int i = 0; i < HB; ++i) Dh[i] = Dp[h0 + i];
  const int nchunks = (si.z + kQ - 1) / kQ;
  const Lofs lo = lane_offsets(lane, ph);
  const DmaOfs dof = dma_offsets(lane, w, ld);
  const uint32_t yvoff = 2u * ((uint32_t)c * (uint32_t)Di + 4u * (uint32_t)g);
  bf16_t* const dBC[2] = {sB, sC};

  auto rows_of = [&](int q) { return xbc + (size_t)(si.y + q * kQ) * ld; };
  auto nr_of = [&](int q) { return min(kQ, si.z - q * kQ); };
  auto dt_of = [&](int q) { return dt_bits(dt, si.y + q * kQ, nr_of(q), H, h, lane); };
  auto load = [&](int q) {
    const int nrb = nr_of(q) * (int)ld * 2;
    load_bc<HB, 2>(rows_of(q), nrb, 2u * ld, colBC, dBC, dof, w);
    load_x<HB>(rows_of(q), nrb, 2u * ld, colX, sX, dof, w);
  };

  // the state entering the segment, frame scale 1: zero for a fresh sequence's first
  // segment; the slot itself for a resumed sequence of one segment (each lane reads here
  // and writes at the end the same elements); the previous segment's local state, walked
  // here from its first kept chunk, where the segment-state kernel left it to this kernel
  // (the previous segment then decays by more than e^-60, so that is the whole entering
  // state); else what the pass left at this segment's index (for a first segment, the
  // pass's copy of the slot, which the sequence's last segment overwrites during this launch)
  f32x4 S[2][8];
  const int prev = si.w > 0 ? uniform(sp.seg_start[(size_t)(seg - 1) * H + h0]) : 0;
  if (si.w == 0 && fresh[si.x]) {
#pragma unroll
    for (int t = 0; t < 2; ++t)
#pragma unroll
      for (int nb = 0; nb < 8; ++nb) S[t][nb] = f32x4{0.f, 0.f, 0.f, 0.f};
  } else if (prev & kTailLeft) {
    const int4 sq0 = sp.seg_info[seg - 1];
    walk_local_state(S, xbc, dt, uniform(sq0.y), uniform(sq0.z), prev & (kTailLeft - 1), H, h, A, bias, ld,
                     colBC[0], colX, sB, sX, sD, lo, dof, w, lane, hh, ph);
  } else {
    const float* in = (si.w == 0 && last) ? pool + ((size_t)slots[si.x] * H + h) * (size_t)(kP * kN)
                                          : sp.seg_state + ((size_t)seg * H + h) * (size_t)(kP * kN);
#pragma unroll
    for (int t = 0; t < 2; ++t)
#pragma unroll
      for (int nb = 0; nb < 8; ++nb) S[t][nb] = *reinterpret_cast<const f32x4*>(in + state_elem(ph, t, nb, lane));
  }

  // a segment starting at a positive multiple of snapE rows of its sequence: the state entering
  // it (frame scale 1 here) is the snapshot at that boundary, the sequence's (offset / snapE)-th,
  // after those of the sequences before it (each with (length - 1) / snapE)
  if (snaps) {
    const int off = si.y - uniform(cu[si.x]);
    if (off > 0 && off % snapE == 0) {  // uniform over the workgroup
      int before = 0;
      for (int s2 = (int)threadIdx.x; s2 < si.x; s2 += 256) before += (cu[s2 + 1] - cu[s2] - 1) / snapE;
#pragma unroll
      for (int o = 32; o >= 1; o >>= 1) before += __shfl_xor(before, o, 64);
      if (lane == 0) sRed[w] = before;
      __syncthreads();
      const int idx = uniform(sRed[0] + sRed[1] + sRed[2] + sRed[3]) + off / snapE - 1;
      float* dst = snaps + ((size_t)idx * H + h) * (size_t)(kP * kN);
#pragma unroll
      for (int t = 0; t < 2; ++t)
#pragma unroll
        for (int nb = 0; nb < 8; ++nb) *reinterpret_cast<f32x4*>(dst + state_elem(ph, t, nb, lane)) = S[t][nb];
    }
  }

  float lam = 1.f, lsum = 0.f;
  load(0);
  chunk_decay(sD[0][hh], bf16_to_f32(dt_of(0)), A, bias, nr_of(0), lane, ph, lam, lsum);
  uint32_t dtn = nchunks > 1 ? dt_of(1) : 0u;

  // M^T tile (jb, ib) of head `head` from the G^T tile, in operand order, hi and lo, with D
  // on the diagonal.  gq, cq: the lane's g and c, recomputed per chunk (see opaque).
  auto m_tile = [&](const f32x4& gt, int jb, int ib, int head, const Decay* dc, int gq, int cq) {
    const Decay& d = dc[head];
    float v[4];
    if (jb < ib) {
      const f32x4 ef = *reinterpret_cast<const f32x4*>(&d.ef[16 * jb + 4 * gq]);
      const float er = d.er[jb][16 * ib + cq];
#pragma unroll
      for (int r = 0; r < 4; ++r) v[r] = gt[r] * (ef[r] * er);
    } else {
      const float csi = d.cs[16 * ib + cq];
      const f32x4 csj = *reinterpret_cast<const f32x4*>(&d.cs[16 * jb + 4 * gq]);
      const f32x4 dtj = *reinterpret_cast<const f32x4*>(&d.dt[16 * jb + 4 * gq]);
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const float e = 4 * gq + r == cq ? Dh[head] : 0.f;
        v[r] = 4 * gq + r > cq ? 0.f : fmaf(gt[r], __expf(csi - csj[r]) * dtj[r], e);
      }
    }
    const u32x4 hl = split4(v[0], v[1], v[2], v[3]);
    const int m = jb >> 1, u = m_unit(ib, m);
    if (m_half(ib, m)) {
      sM[head][u][lane] = hl;
    } else {
      u32x2* hp = reinterpret_cast<u32x2*>(&sM[head][u][lane]) + (jb & 1);
      hp[0] = u32x2{hl[0], hl[1]};
      hp[128] = u32x2{hl[2], hl[3]};  // the lo unit, 64 lanes x 16 bytes further
    }
  };

  for (int q = 0; q < nchunks; ++q) {
    const int r0 = si.y + q * kQ;
    const int nr = nr_of(q);
    const Decay* dc = sD[q & 1];
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();  // (1) chunk q tiles and decay visible; chunk q-1 done with M
    const int gq = opaque(g), cq = opaque(c);

    // ---- phase 1: x operands; G^T tiles and M^T for the workgroup's heads; S C^T; state ----
    u32x4 xt[2][2];
#pragma unroll
    for (int t = 0; t < 2; ++t)
#pragma unroll
      for (int m = 0; m < 2; ++m) xt[t][m] = tr_frag<kP>(sX[hh] + lo.xt[t], m);

    auto gt_tile = [&](int jb, int ib) {
      f32x4 acc = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int kk = 0; kk < 4; ++kk)
        acc = mfma(lds16(sB + (lo.gt[kk & 1] ^ (64 * (kk >> 1))) + 16 * jb * kN),
                   lds16(sC + (lo.gt[kk & 1] ^ (64 * (kk >> 1))) + 16 * ib * kN), acc);
      return acc;
    };
    // tiles 0..7 for every head, one per wave (two per wave with four waves); tiles
    // 8 = (2, 3) and 9 = (3, 3) for the wave's own head.  Instantiated per wave index, so
    // every tile position and weight form is fixed at compile time (one uniform branch).
    auto wave_tiles = [&](auto wc) {
      constexpr int W = decltype(wc)::value;
#pragma unroll
      for (int i = 0; i < 8 / (2 * HB); ++i) {
        const int t = W + 2 * HB * i;
        const int ib = t < 1 ? 0 : t < 3 ? 1 : t < 6 ? 2 : 3;
        const int jb = t - ib * (ib + 1) / 2;
        const f32x4 gt = gt_tile(jb, ib);
#pragma unroll
        for (int head = 0; head < HB; ++head) m_tile(gt, jb, ib, head, dc, gq, cq);
      }
      if ((W & 1) == 0) m_tile(gt_tile(2, 3), 2, 3, W >> 1, dc, gq, cq);
      else m_tile(gt_tile(3, 3), 3, 3, W >> 1, dc, gq, cq);
    };
    static_assert(2 * HB <= 8, "wave dispatch");
    auto wave_case = [&](auto wc) {
      if constexpr (decltype(wc)::value < 2 * HB) wave_tiles(wc);
    };
    switch (w) {
      case 0: wave_case(std::integral_constant<int, 0>{}); break;
      case 1: wave_case(std::integral_constant<int, 1>{}); break;
      case 2: wave_case(std::integral_constant<int, 2>{}); break;
      case 3: wave_case(std::integral_constant<int, 3>{}); break;
      case 4: wave_case(std::integral_constant<int, 4>{}); break;
      case 5: wave_case(std::integral_constant<int, 5>{}); break;
      case 6: wave_case(std::integral_constant<int, 6>{}); break;
      default: wave_case(std::integral_constant<int, 7>{}); break;
    }

    // Y^T(pb, ib) = S C^T, the state operand split from the accumulators; then the update.
    // The MFMA-heavy stretch runs at raised wave priority so that the SIMD's other wave fills
    // the matrix core's gaps with its vector work rather than the reverse.
    __builtin_amdgcn_s_setprio(1);
    __builtin_amdgcn_iglp_opt(1);  // interleave the splits' vector work with the MFMAs
    const Decay& d = dc[hh];
    f32x4 Y[2][4];
#pragma unroll
    for (int t = 0; t < 2; ++t)
#pragma unroll
      for (int ib = 0; ib < 4; ++ib) Y[t][ib] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) {
      u32x4 sh[2], sl[2];
#pragma unroll
      for (int t = 0; t < 2; ++t) {
        const f32x4 a = S[t][2 * kk], b = S[t][2 * kk + 1];
        const u32x4 sa = split4(a[0], a[1], a[2], a[3]), sb = split4(b[0], b[1], b[2], b[3]);
        sh[t] = u32x4{sa[0], sa[1], sb[0], sb[1]};
        sl[t] = u32x4{sa[2], sa[3], sb[2], sb[3]};
      }
#pragma unroll
      for (int ib = 0; ib < 4; ++ib) {
        const u32x4 cf = lds16(sC + 16 * ib * kN + lo.cf[kk]);
#pragma unroll
        for (int t = 0; t < 2; ++t) {
          Y[t][ib] = mfma(sh[t], cf, Y[t][ib]);
          Y[t][ib] = mfma(sl[t], cf, Y[t][ib]);
        }
      }
    }
    state_update(S, xt, sB, lo, d, lane);
    __builtin_amdgcn_s_setprio(0);
    float ei[4];
#pragma unroll
    for (int ib = 0; ib < 4; ++ib) ei[ib] = d.e[16 * ib + cq];
#pragma unroll
    for (int t = 0; t < 2; ++t)
#pragma unroll
      for (int ib = 0; ib < 4; ++ib) Y[t][ib] *= ei[ib];
    __syncthreads();  // (2) M^T visible; the tiles of chunk q no longer read

    uint32_t dtn2 = 0;
    if (q + 1 < nchunks) {
      load(q + 1);
      if (q + 2 < nchunks) dtn2 = dt_of(q + 2);
    }

    // ---- phase 2: + x^T M^T (D x on its diagonal), row scales, store ----
#pragma unroll
    for (int ib = 0; ib < 4; ++ib) {
#pragma unroll
      for (int m = 0; m < 2; ++m) {
        if (m <= (ib >> 1)) {
          u32x4 mh, ml;
          if (m_half(ib, m)) {
            const u32x4 t0 = sM[hh][m_unit(ib, m)][lane];
            mh = u32x4{t0[0], t0[1], 0u, 0u};
            ml = u32x4{t0[2], t0[3], 0u, 0u};
          } else {
            mh = sM[hh][m_unit(ib, m)][lane];
            ml = sM[hh][m_unit(ib, m) + 1][lane];
          }
#pragma unroll
          for (int t = 0; t < 2; ++t) {
            Y[t][ib] = mfma(xt[t][m], mh, Y[t][ib]);
            Y[t][ib] = mfma(xt[t][m], ml, Y[t][ib]);
          }
        }
      }
    }
#pragma unroll
    for (int ib = 0; ib < 4; ++ib) {
      // rows 16 ib.. of the chunk; rows at or past nr are dropped by the range
      const Rsrc yr = make_rsrc(y + (size_t)(r0 + 16 * ib) * Di, ((int64_t)nr - 16 * ib) * Di * 2);
#pragma unroll
      for (int t = 0; t < 2; ++t) {
        const f32x4 o = Y[t][ib];
        bst8(yr, yvoff, 2u * (uint32_t)(h * kP + 32 * ph + 16 * t), u32x2{pk(o[0], o[1]), pk(o[2], o[3])});
      }
    }
    if (q + 1 < nchunks) chunk_decay(sD[(q + 1) & 1][hh], bf16_to_f32(dtn), A, bias, nr_of(q + 1), lane, ph, lam, lsum);
    dtn = dtn2;
  }
  if (last) {
    const float lam_end = uniformf(sD[(nchunks - 1) & 1][hh].lam_next);
    float* out = pool + ((size_t)slots[si.x] * H + h) * (size_t)(kP * kN);
    const int lane_st = opaque(lane);
#pragma unroll
    for (int t = 0; t < 2; ++t)
#pragma unroll
      for (int nb = 0; nb < 8; ++nb)
        *reinterpret_cast<f32x4*>(out + state_elem(ph, t, nb, lane_st)) = S[t][nb] * lam_end;
  }
}

constexpr int kHeadsPerBlock = 2;

}  // namespace

// Shapes the MFMA path covers: bf16, P = 64, N = 128, an even number of heads per group
// (a workgroup takes 2 heads of one group), and chunk-row offsets within 32 bits.
bool scan_mfma_supported(const mamba2_dims* d) {
  const int64_t Dc = (int64_t)d->nheads * d->headdim + 2 * (int64_t)d->ngroups * d->d_state;
  return d->act_dtype == MAMBA2_DTYPE_BF16 && d->headdim == kP && d->d_state == kN &&
         (d->nheads / d->ngroups) % 2 == 0 && Dc * kQ * 2 < ((int64_t)1 << 31);
}

// Segment length for the MFMA path: aim at three rounds of workgroups (two resident per CU
// on each of 256 CUs), 64..4096 rows per segment.
int32_t scan_mfma_segment_length(const mamba2_recurrent_batch* rb, const mamba2_dims* d) {
  const int64_t groups = d->nheads / kHeadsPerBlock;
  const int64_t target = 3 * 512;
  int64_t L = ((int64_t)rb->num_rows * groups + target - 1) / target;
  L = (L + kQ - 1) / kQ * kQ;
  if (L < kQ) L = kQ;
  if (L > 4096) L = 4096;
  return (int32_t)L;
}

hipError_t launch_scan_mfma(const ScanArgs& a, hipStream_t st) {
  const SegPtrs sp{(const int2*)(a.ws + a.lay.off_seq_info), (const int4*)(a.ws + a.lay.off_seg_info),
                   (float*)(a.ws + a.lay.off_seg_decay), (float*)(a.ws + a.lay.off_seg_state),
                   (int*)(a.ws + a.lay.off_seg_start), (float*)(a.ws + a.lay.off_seg_chunk),
                   a.keep_seg_states ? 0 : 1};
  const mamba2_dims& d = a.dims;
  const int nitems = (int)(a.lay.nseg * (d.nheads / kHeadsPerBlock));
  if (nitems == 0) return hipSuccess;
  if (a.lay.seg_len > kMaxSegChunks * kQ) return hipErrorInvalidValue;  // the chunk-sum table
  const int cpb = (a.lay.seg_len + kQ - 1) / kQ;  // one workgroup per chunk of a segment
  const dim3 sums_grid((unsigned)(a.lay.nseg * cpb));
  int2* seq_out = (int2*)(a.ws + a.lay.off_seq_info);
  int4* seg_out = (int4*)(a.ws + a.lay.off_seg_info);
  if (a.bd.num_seqs <= kTableSeqs) {
    M2_LAUNCH("chunk_sums", chunk_sums_kernel<true>, sums_grid, dim3(256), 0, st, (const bf16_t*)a.dt, a.a_log,
              a.dt_bias, sp, d.nheads, cpb, a.bd.cu_seqlens, a.bd.num_seqs, a.lay.seg_len, seq_out, seg_out);
  } else {
    hipError_t e = launch_scan_setup(a, st);
    if (e != hipSuccess) return e;
    M2_LAUNCH("chunk_sums", chunk_sums_kernel<false>, sums_grid, dim3(256), 0, st, (const bf16_t*)a.dt, a.a_log,
              a.dt_bias, sp, d.nheads, cpb, a.bd.cu_seqlens, a.bd.num_seqs, a.lay.seg_len, seq_out, seg_out);
  }
  M2_LAUNCH("ssd_state", ssd_state_kernel, dim3((unsigned)nitems), dim3(256), 0, st, (const bf16_t*)a.xbc,
            (const bf16_t*)a.dt, a.a_log, a.dt_bias, sp, d.nheads, d.ngroups, nitems);
  hipError_t e = launch_scan_pass(a, st);
  if (e != hipSuccess) return e;
  M2_LAUNCH("ssd_scan", ssd_scan_kernel, dim3((unsigned)nitems), dim3(256), 0, st, (bf16_t*)a.y,
            (const bf16_t*)a.xbc, (const bf16_t*)a.dt, a.a_log, a.dt_bias, a.D, a.ssm_state, a.bd.slots,
            a.bd.fresh, sp, d.nheads, d.ngroups, nitems, a.bd.cu_seqlens, a.snaps, a.snap_every);
  return hipSuccess;
}

}  // namespace m2
