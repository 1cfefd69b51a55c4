// Chunked selective scan for prefill: segment tables and the inter-segment state pass.
//
// The chunked form of the recurrence ("feat(backend): Mamba2 ops, with CPU reference
// implementations", section "Ops", SSMScan; "Granite Mamba2 Inference Optimization":
// long prefill as a chunked parallel scan).  Each sequence is cut into segments of
// seg_len rows aligned to its first row, so no segment spans two sequences and the
// state never crosses a sequence boundary.  With a_t = -exp(A_log) * dt'_t and
// S_in(k) the state entering segment k of a sequence:
//   S_in(0)   = 0 when fresh, else the slot,
//   S_in(k+1) = exp(sum_{t in k} a_t) * S_in(k) + S_loc(k),
//   S_loc(k)  = sum_{j in k} exp(sum_{t in k, t > j} a_t) * dt'_j * x_j (x) B_j.
// Three launches: segment states S_loc(k) for every segment but a sequence's last
// (scan kernels; stored at the index of segment k + 1, with the segment's decay factor),
// this pass (turns them into S_in, serially over a sequence's segments), and the output
// kernels that walk each segment from S_in, write y and, for a sequence's last segment,
// the final state into the slot.
//
// A carried state whose decay to the point of use is below e^-60 is dropped: its share is
// below fp32 resolution next to the terms that are kept.  A segment whose whole decay is
// that small has decay factor 0 and S_in(k+1) = S_loc(k): the pass leaves its slot as the
// scan kernel wrote it and, where every segment decays that much, moves no state at all.
#include "common.h"

namespace m2 {

namespace {

constexpr int kSetupThreads = 1024;

__global__ __launch_bounds__(kSetupThreads) void scan_setup_kernel(const int32_t* __restrict__ cu,
                                                                   int S, int seg_len,
                                                                   int2* __restrict__ seq_info,
                                                                   int4* __restrict__ seg_info) {
  __shared__ int buf[kSetupThreads];
  __shared__ int carry;
  const int tid = threadIdx.x;
  if (tid == 0) carry = 0;
  __syncthreads();
  for (int base = 0; base < S; base += kSetupThreads) {
    const int s = base + tid;
    int len = 0, n = 0;
    if (s < S) {
      len = cu[s + 1] - cu[s];
      n = (len + seg_len - 1) / seg_len;
    }
    buf[tid] = n;
    __syncthreads();
    for (int o = 1; o < kSetupThreads; o <<= 1) {
      const int add = tid >= o ? buf[tid - o] : 0;
      __syncthreads();
      buf[tid] += add;
      __syncthreads();
    }
    const int first = carry + buf[tid] - n;
    if (s < S) {
      seq_info[s] = make_int2(first, n);
      for (int k = 0; k < n; ++k)
        seg_info[first + k] = make_int4(s, cu[s] + k * seg_len, min(seg_len, len - k * seg_len), k);
    }
    __syncthreads();
    if (tid == kSetupThreads - 1) carry += buf[tid];
    __syncthreads();
  }
}

// One thread per float4 of a head's state, walking one sequence's segments in order
// (sequences strided over grid z).  Index k > 0 of a sequence's state array holds S_loc(k - 1)
// as the scan kernels left it; where segment k - 1 has a nonzero decay factor the pass
// replaces it with S_in(k) = dec(k - 1) S_in(k - 1) + S_loc(k - 1).  S_in(k - 1) is in the
// registers when the previous step computed it, else it is read back from index k - 1 (a
// dropped predecessor: S_loc(k - 2)).  A resumed sequence of several segments has its slot
// copied to index 0, since the launch that reads S_in(0) also writes the final state into
// that slot.  The decays and the local states of kBatch segments are loaded before the chain
// runs through them, so a long chain waits on one round of loads per batch rather than one
// per segment.
constexpr int kBatch = 8;

__global__ __launch_bounds__(256) void scan_pass_kernel(const int2* __restrict__ seq_info,
                                                        const float* __restrict__ seg_decay,
                                                        float4* __restrict__ seg_state,
                                                        const float4* __restrict__ pool,
                                                        const int32_t* __restrict__ slots,
                                                        const uint8_t* __restrict__ fresh, int H,
                                                        int f4, int S) {
  const int f = blockIdx.x * blockDim.x + threadIdx.x;
  const int h = blockIdx.y;
  const bool live = f < f4;  // lanes past the state only take part in the wave's test below
  for (int s = blockIdx.z; s < S; s += gridDim.z) {
    const int2 si = seq_info[s];
    if (si.y < 2) continue;
    auto at = [&](int k) -> float4& { return seg_state[((size_t)(si.x + k) * H + h) * f4 + f]; };
    float4 Sr = make_float4(0.f, 0.f, 0.f, 0.f);
    if (live && !fresh[s]) {
      Sr = pool[((size_t)slots[s] * H + h) * f4 + f];
      at(0) = Sr;
    }
    // no segment with a nonzero factor (every carried state dropped): nothing to chain.  All
    // 64 lanes of the wave read the factors, 64 at a time, so the wave leaves after one round
    bool any = false;
    for (int k0 = 0; k0 + 1 < si.y && !any; k0 += 64) {
      const int k = k0 + (int)(threadIdx.x & 63);
      any = __ballot(k + 1 < si.y && seg_decay[(int64_t)(si.x + k) * H + h] != 0.f) != 0;
    }
    if (!any || !live) continue;
    bool valid = true;  // Sr holds S_in(k) of the step below
    for (int k0 = 0; k0 + 1 < si.y; k0 += kBatch) {
      float4 loc[kBatch];
      float dec[kBatch];
#pragma unroll
      for (int i = 0; i < kBatch; ++i) {
        const int k = k0 + i;
        dec[i] = k + 1 < si.y ? seg_decay[(int64_t)(si.x + k) * H + h] : 0.f;
        loc[i] = dec[i] != 0.f ? at(k + 1) : make_float4(0.f, 0.f, 0.f, 0.f);
      }
#pragma unroll
      for (int i = 0; i < kBatch; ++i) {
        const int k = k0 + i;
        if (k + 1 < si.y && dec[i] != 0.f) {
          if (!valid) Sr = at(k);
          Sr.x = fmaf(dec[i], Sr.x, loc[i].x);
          Sr.y = fmaf(dec[i], Sr.y, loc[i].y);
          Sr.z = fmaf(dec[i], Sr.z, loc[i].z);
          Sr.w = fmaf(dec[i], Sr.w, loc[i].w);
          at(k + 1) = Sr;  // S_in(k + 1)
          valid = true;
        } else {
          valid = false;
        }
      }
    }
  }
}

size_t align256(size_t v) { return (v + 255) & ~(size_t)255; }

}  // namespace

bool scan_mfma_supported(const mamba2_dims* d);
int32_t scan_mfma_segment_length(const mamba2_recurrent_batch* rb, const mamba2_dims* d);

bool scan_uses_mfma(const mamba2_dims* d) { return scan_mfma_supported(d); }

int32_t scan_segment_length(const mamba2_recurrent_batch* rb, const mamba2_dims* d, bool mfma) {
  if (!mfma) {
    const int q = d->chunk_size < 64 ? d->chunk_size : 64;
    return q < 1 ? 1 : q;
  }
  return scan_mfma_segment_length(rb, d);
}

// With snapshots every E rows, segments must start at every multiple of E: the longest
// segment length that divides E, is a multiple of the path's unit (the chunk of the MFMA
// path, the one-chunk segment of the generic path) and is at most the usual length.
int32_t scan_segment_length_snap(const mamba2_recurrent_batch* rb, const mamba2_dims* d, int32_t E) {
  const bool mfma = scan_uses_mfma(d);
  const int32_t usual = scan_segment_length(rb, d, mfma);
  const int32_t unit = mfma ? 64 : scan_segment_length(rb, d, false);
  if (E < 1 || E % unit != 0) return 0;
  int32_t best = unit;
  for (int32_t k = 1; (int64_t)k * unit <= usual; ++k)
    if ((E / unit) % k == 0) best = k * unit;
  return best;
}

ScanLayout scan_layout(const mamba2_recurrent_batch* rb, const mamba2_dims* d, int32_t seg_len) {
  ScanLayout L{};
  L.seg_len = seg_len;
  int64_t nseg = 0;
  for (int s = 0; s < rb->num_seqs; ++s) nseg += (rb->run_lengths[s] + seg_len - 1) / seg_len;
  L.nseg = nseg;
  const size_t S = (size_t)rb->num_seqs;
  const size_t H = (size_t)d->nheads;
  const size_t PN = (size_t)d->headdim * d->d_state;
  size_t off = 0;
  L.off_seq_info = off;
  off = align256(off + S * sizeof(int2));
  L.off_seg_info = off;
  off = align256(off + (size_t)nseg * sizeof(int4));
  L.off_seg_decay = off;
  off = align256(off + (size_t)nseg * H * sizeof(float));
  L.off_seg_start = off;
  off = align256(off + (size_t)nseg * H * sizeof(int32_t));
  L.off_seg_chunk = off;
  off = align256(off + (size_t)nseg * 64 * H * sizeof(float));
  L.off_seg_state = off;
  off = align256(off + (size_t)nseg * H * PN * sizeof(float));
  L.total = off;
  return L;
}

// Sequence and segment tables of any packed batch (also the chunk tables of the Mamba-3
// forward): seq_info [S], seg_info [number of segments].
hipError_t launch_segment_tables(const int32_t* cu, int S, int seg_len, int2* seq_info, int4* seg_info,
                                 hipStream_t st) {
  M2_LAUNCH("scan_setup", scan_setup_kernel, dim3(1), dim3(kSetupThreads), 0, st, cu, S, seg_len, seq_info, seg_info);
  return hipSuccess;
}

hipError_t launch_scan_setup(const ScanArgs& a, hipStream_t st) {
  M2_LAUNCH("scan_setup", scan_setup_kernel, dim3(1), dim3(kSetupThreads), 0, st, a.bd.cu_seqlens,
            a.bd.num_seqs, a.lay.seg_len, (int2*)(a.ws + a.lay.off_seq_info),
            (int4*)(a.ws + a.lay.off_seg_info));
  return hipSuccess;
}

hipError_t launch_scan_pass(const ScanArgs& a, hipStream_t st) {
  const int f4 = a.dims.headdim * a.dims.d_state / 4;
  const int S = a.bd.num_seqs;
  const dim3 grid((unsigned)((f4 + 255) / 256), (unsigned)a.dims.nheads, (unsigned)(S < 65535 ? S : 65535));
  M2_LAUNCH("scan_pass", scan_pass_kernel, grid, dim3(256), 0, st,
            (const int2*)(a.ws + a.lay.off_seq_info), (const float*)(a.ws + a.lay.off_seg_decay),
            (float4*)(a.ws + a.lay.off_seg_state), (const float4*)a.ssm_state, a.bd.slots,
            a.bd.fresh, a.dims.nheads, f4, S);
  return hipSuccess;
}

hipError_t launch_scan_generic(const ScanArgs& a, hipStream_t st);
hipError_t launch_scan_mfma(const ScanArgs& a, hipStream_t st);

hipError_t launch_scan_prefill(const ScanArgs& a, hipStream_t st) {
  if (scan_uses_mfma(&a.dims)) return launch_scan_mfma(a, st);  // builds the tables itself
  hipError_t e = launch_scan_setup(a, st);
  if (e != hipSuccess) return e;
  return launch_scan_generic(a, st);
}

}  // namespace m2
