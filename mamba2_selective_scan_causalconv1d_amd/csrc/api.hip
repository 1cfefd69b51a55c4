// C ABI of the Mamba2 mixer hot path: host-side validation and kernel launches.
//
// Every check runs before the first launch; on any error nothing is enqueued and
// nothing is written.  The library allocates no device memory and never
// synchronises the host with the stream.
#include <algorithm>
#include <initializer_list>
#include <mutex>
#include <vector>

#include "common.h"

using namespace m2;

// Scratch of mamba2_scan_prefill_static: the chunked scan's workspace for callers that cannot
// allocate.  Each GPU the library runs on holds its own copy until the process ends.  In host
// code this name stands for the array, not for its device address: the address comes from
// hipGetSymbolAddress, per device (static_scratch below).
constexpr size_t kStaticScratchBytes = (size_t)32 << 20;
static __device__ __align__(256) char scratch[kStaticScratchBytes];

namespace {

constexpr int64_t kMaxElems = (int64_t)1 << 31;

mamba2_status check_dims(const mamba2_dims* d) {
  if (!d) return MAMBA2_INVALID_ARGUMENT;
  if (d->nheads < 1 || d->headdim < 1 || d->d_state < 1 || d->ngroups < 1) return MAMBA2_INVALID_ARGUMENT;
  if (d->nheads % d->ngroups != 0) return MAMBA2_INVALID_ARGUMENT;
  if (d->conv_kernel < 1 || d->chunk_size < 1 || d->pool_slots < 0) return MAMBA2_INVALID_ARGUMENT;
  if (d->act_dtype != MAMBA2_DTYPE_F32 && d->act_dtype != MAMBA2_DTYPE_BF16) return MAMBA2_INVALID_ARGUMENT;
  const int64_t Di = (int64_t)d->nheads * d->headdim;
  const int64_t Dc = Di + 2 * (int64_t)d->ngroups * d->d_state;
  const int64_t hpn = Di * d->d_state;
  if (Dc >= kMaxElems || hpn >= kMaxElems) return MAMBA2_INVALID_ARGUMENT;
  return MAMBA2_OK;
}

// Run lengths, then slot range, then slot sharing (the RecurrentBatch rules).
mamba2_status check_batch(const mamba2_recurrent_batch* rb, const mamba2_dims* d, bool decode) {
  if (!rb) return MAMBA2_INVALID_ARGUMENT;
  const int S = rb->num_seqs;
  if (S < 0 || rb->num_rows < 0) return MAMBA2_INVALID_ARGUMENT;
  if (S > 0 && (!rb->run_lengths || !rb->slots || !rb->fresh || !rb->dev_cu_seqlens ||
                !rb->dev_slots || !rb->dev_fresh))
    return MAMBA2_INVALID_ARGUMENT;
  int64_t sum = 0;
  for (int s = 0; s < S; ++s) {
    const int32_t L = rb->run_lengths[s];
    if (L <= 0 || (decode && L != 1)) return MAMBA2_RUN_LENGTHS;
    sum += L;
  }
  if (sum != rb->num_rows) return MAMBA2_RUN_LENGTHS;
  for (int s = 0; s < S; ++s)
    if (rb->slots[s] < 0 || rb->slots[s] >= d->pool_slots) return MAMBA2_SLOT_OUT_OF_RANGE;
  if (S > 1) {
    std::vector<int32_t> v(rb->slots, rb->slots + S);
    std::sort(v.begin(), v.end());
    for (int s = 1; s < S; ++s)
      if (v[s] == v[s - 1]) return MAMBA2_SLOT_SHARED;
  }
  return MAMBA2_OK;
}

// The kernels move activations, states and weight vectors in 16-byte units.
bool aligned16(std::initializer_list<const void*> ps) {
  for (const void* p : ps)
    if (((uintptr_t)p & 15) != 0) return false;
  return true;
}

mamba2_status check_all(const mamba2_recurrent_batch* rb, const mamba2_dims* d, bool decode) {
  mamba2_status st = check_dims(d);
  if (st != MAMBA2_OK) return st;
  return check_batch(rb, d, decode);
}

int act_vec(int32_t act) { return act == MAMBA2_DTYPE_BF16 ? 8 : 4; }

BatchDev batch_dev(const mamba2_recurrent_batch* rb) {
  return BatchDev{rb->dev_cu_seqlens, rb->dev_slots, rb->dev_fresh, rb->num_seqs, rb->num_rows};
}

mamba2_status from_hip(hipError_t e) { return e == hipSuccess ? MAMBA2_OK : MAMBA2_HIP_ERROR; }

// Device address of the current device's scratch array, looked up once per device with that
// device current; null if the lookup fails.
char* static_scratch() {
  constexpr int kMaxDevices = 64;
  static std::mutex mu;
  static char* ptr[kMaxDevices] = {};
  static bool done[kMaxDevices] = {};
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return nullptr;
  std::lock_guard<std::mutex> lock(mu);
  if (!done[dev]) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess) p = nullptr;
    ptr[dev] = (char*)p;
    done[dev] = p != nullptr;
  }
  return ptr[dev];
}

// Shapes the prefill scan covers (both paths need N % 4 == 0 for 16-byte state access).
bool scan_supported(const mamba2_dims* d) { return d->d_state % 4 == 0; }

mamba2_status padded_call(bool pack, void* dst, const void* src, int64_t row_bytes, int32_t max_len,
                          int32_t left_padded, const mamba2_recurrent_batch* rb, void* stream) {
  if (!rb || row_bytes < 1 || max_len < 1 || (left_padded != 0 && left_padded != 1)) return MAMBA2_INVALID_ARGUMENT;
  const int S = rb->num_seqs;
  if (S < 0 || rb->num_rows < 0) return MAMBA2_INVALID_ARGUMENT;
  if (S > 0 && (!rb->run_lengths || !rb->dev_cu_seqlens || !dst || !src)) return MAMBA2_INVALID_ARGUMENT;
  int64_t sum = 0;
  for (int s = 0; s < S; ++s) {
    if (rb->run_lengths[s] < 1 || rb->run_lengths[s] > max_len) return MAMBA2_RUN_LENGTHS;
    sum += rb->run_lengths[s];
  }
  if (sum != rb->num_rows) return MAMBA2_RUN_LENGTHS;
  if ((int64_t)S * max_len * row_bytes >= ((int64_t)1 << 46)) return MAMBA2_INVALID_ARGUMENT;
  if (S == 0) return MAMBA2_OK;
  return from_hip(launch_padded(pack, dst, src, batch_dev(rb), max_len, left_padded, row_bytes,
                                (hipStream_t)stream));
}

}  // namespace

extern "C" {

mamba2_status mamba2_validate(const mamba2_recurrent_batch* rb, const mamba2_dims* dims,
                              int32_t decode) {
  return check_all(rb, dims, decode != 0);
}

mamba2_status mamba2_conv1d(void* dst, const void* x, const float* weight, const float* bias,
                            void* conv_state, const mamba2_recurrent_batch* rb,
                            const mamba2_dims* dims, void* stream) {
  mamba2_status st = check_dims(dims);
  if (st != MAMBA2_OK) return st;
  if (!rb) return MAMBA2_INVALID_ARGUMENT;
  if (rb->num_rows > 0 && (!dst || !x || !weight || !bias || !conv_state)) return MAMBA2_INVALID_ARGUMENT;
  if (!aligned16({dst, x, weight, bias, conv_state})) return MAMBA2_INVALID_ARGUMENT;
  st = check_batch(rb, dims, false);
  if (st != MAMBA2_OK) return st;
  const int64_t Dc = (int64_t)dims->nheads * dims->headdim + 2 * (int64_t)dims->ngroups * dims->d_state;
  if (dims->conv_kernel < 2 || dims->conv_kernel > 4 || Dc % act_vec(dims->act_dtype) != 0)
    return MAMBA2_NOT_IMPLEMENTED;
  if (rb->num_rows == 0) return MAMBA2_OK;
  return from_hip(launch_conv1d(dst, x, weight, bias, conv_state, batch_dev(rb), (int32_t)Dc,
                                dims->conv_kernel, dims->act_dtype, (hipStream_t)stream));
}

size_t mamba2_scan_prefill_workspace_bytes(const mamba2_recurrent_batch* rb, const mamba2_dims* dims) {
  if (check_all(rb, dims, false) != MAMBA2_OK || rb->num_rows == 0) return 0;
  const bool mfma = scan_uses_mfma(dims);
  return scan_layout(rb, dims, scan_segment_length(rb, dims, mfma)).total;
}

mamba2_status mamba2_scan_prefill(void* dst, const void* xbc, const void* dt, const float* a_log,
                                  const float* dt_bias, const float* d, float* ssm_state,
                                  const mamba2_recurrent_batch* rb, const mamba2_dims* dims,
                                  void* workspace, size_t workspace_bytes, void* stream) {
  mamba2_status st = check_dims(dims);
  if (st != MAMBA2_OK) return st;
  if (!rb) return MAMBA2_INVALID_ARGUMENT;
  if (rb->num_rows > 0 && (!dst || !xbc || !dt || !a_log || !dt_bias || !d || !ssm_state))
    return MAMBA2_INVALID_ARGUMENT;
  if (!aligned16({dst, xbc, ssm_state})) return MAMBA2_INVALID_ARGUMENT;
  st = check_batch(rb, dims, false);
  if (st != MAMBA2_OK) return st;
  if (!scan_supported(dims)) return MAMBA2_NOT_IMPLEMENTED;
  if (rb->num_rows == 0) return MAMBA2_OK;
  const bool mfma = scan_uses_mfma(dims);
  const ScanLayout lay = scan_layout(rb, dims, scan_segment_length(rb, dims, mfma));
  if (!workspace || workspace_bytes < lay.total) return MAMBA2_WORKSPACE_TOO_SMALL;
  if (((uintptr_t)workspace & 255) != 0) return MAMBA2_INVALID_ARGUMENT;
  ScanArgs a{dst, xbc, dt, a_log, dt_bias, d, ssm_state, batch_dev(rb), *dims, lay, (char*)workspace, false, nullptr, 0};
  return from_hip(launch_scan_prefill(a, (hipStream_t)stream));
}

mamba2_status mamba2_scan_prefill_static(void* dst, const void* xbc, const void* dt, const float* a_log,
                                         const float* dt_bias, const float* d, float* ssm_state,
                                         const mamba2_recurrent_batch* rb, const mamba2_dims* dims, void* stream) {
  mamba2_status st = check_dims(dims);
  if (st != MAMBA2_OK) return st;
  if (!rb) return MAMBA2_INVALID_ARGUMENT;
  if (rb->num_rows > 0 && (!dst || !xbc || !dt || !a_log || !dt_bias || !d || !ssm_state))
    return MAMBA2_INVALID_ARGUMENT;
  if (!aligned16({dst, xbc, ssm_state})) return MAMBA2_INVALID_ARGUMENT;
  st = check_batch(rb, dims, false);
  if (st != MAMBA2_OK) return st;
  if (!scan_supported(dims)) return MAMBA2_NOT_IMPLEMENTED;
  if (rb->num_rows == 0) return MAMBA2_OK;
  // the usual segment length if its workspace fits the scratch, else longer segments (fewer
  // segment states) on the MFMA path, up to its longest
  const bool mfma = scan_uses_mfma(dims);
  int32_t L = scan_segment_length(rb, dims, mfma);
  ScanLayout lay = scan_layout(rb, dims, L);
  while (lay.total > kStaticScratchBytes && mfma && L < 4096) {
    L = std::min<int32_t>(4096, 2 * L);
    lay = scan_layout(rb, dims, L);
  }
  if (lay.total > kStaticScratchBytes) return MAMBA2_WORKSPACE_TOO_SMALL;
  char* ws = static_scratch();
  if (!ws) return MAMBA2_HIP_ERROR;
  ScanArgs a{dst, xbc, dt, a_log, dt_bias, d, ssm_state, batch_dev(rb), *dims, lay, ws, false, nullptr, 0};
  return from_hip(launch_scan_prefill(a, (hipStream_t)stream));
}

mamba2_status mamba2_scan_decode(void* dst, const void* xbc, const void* dt, const float* a_log,
                                 const float* dt_bias, const float* d, float* ssm_state,
                                 const mamba2_recurrent_batch* rb, const mamba2_dims* dims,
                                 void* stream) {
  mamba2_status st = check_dims(dims);
  if (st != MAMBA2_OK) return st;
  if (!rb) return MAMBA2_INVALID_ARGUMENT;
  if (rb->num_rows > 0 && (!dst || !xbc || !dt || !a_log || !dt_bias || !d || !ssm_state))
    return MAMBA2_INVALID_ARGUMENT;
  if (!aligned16({dst, xbc, ssm_state})) return MAMBA2_INVALID_ARGUMENT;
  st = check_batch(rb, dims, true);
  if (st != MAMBA2_OK) return st;
  if (!decode_supported(*dims) || !decode_grid_fits(*dims, rb->num_seqs)) return MAMBA2_NOT_IMPLEMENTED;
  if (rb->num_rows == 0) return MAMBA2_OK;
  return from_hip(launch_scan_decode(dst, xbc, dt, a_log, dt_bias, d, ssm_state, batch_dev(rb), *dims,
                                     (hipStream_t)stream));
}

mamba2_status mamba2_gated_rmsnorm(void* dst, const void* x, const void* z, const float* weight,
                                   int32_t groups, float eps, int32_t rows, int32_t d_inner,
                                   int32_t act_dtype, void* stream) {
  if (rows < 0 || d_inner < 1 || groups < 1 || d_inner % groups != 0) return MAMBA2_INVALID_ARGUMENT;
  if (act_dtype != MAMBA2_DTYPE_F32 && act_dtype != MAMBA2_DTYPE_BF16) return MAMBA2_INVALID_ARGUMENT;
  if (!(eps >= 0.f) || eps == __builtin_inff()) return MAMBA2_INVALID_ARGUMENT;
  if (rows > 0 && (!dst || !x || !z || !weight)) return MAMBA2_INVALID_ARGUMENT;
  if (!aligned16({dst, x, z, weight})) return MAMBA2_INVALID_ARGUMENT;
  if ((int64_t)rows * d_inner >= ((int64_t)1 << 40)) return MAMBA2_INVALID_ARGUMENT;
  if ((d_inner / groups) % act_vec(act_dtype) != 0) return MAMBA2_NOT_IMPLEMENTED;
  if (rows == 0) return MAMBA2_OK;
  return from_hip(launch_gated_rmsnorm(dst, x, z, weight, groups, eps, rows, d_inner, act_dtype,
                                       (hipStream_t)stream));
}

int64_t mamba2_snapshot_count(const mamba2_recurrent_batch* rb, int32_t snap_every) {
  if (!rb || snap_every < 1 || rb->num_seqs < 0 || (rb->num_seqs > 0 && !rb->run_lengths)) return -1;
  for (int s = 0; s < rb->num_seqs; ++s)
    if (rb->run_lengths[s] < 1) return -1;
  return snapshot_count(rb, snap_every);
}

mamba2_status mamba2_conv1d_snap(void* dst, const void* x, const float* weight, const float* bias,
                                 void* conv_state, void* conv_snaps, int32_t snap_every,
                                 const mamba2_recurrent_batch* rb, const mamba2_dims* dims, void* stream) {
  mamba2_status st = check_dims(dims);
  if (st != MAMBA2_OK) return st;
  if (!rb || snap_every < 1) return MAMBA2_INVALID_ARGUMENT;
  if (rb->num_rows > 0 && (!dst || !x || !weight || !bias || !conv_state)) return MAMBA2_INVALID_ARGUMENT;
  if (!aligned16({dst, x, weight, bias, conv_state, conv_snaps})) return MAMBA2_INVALID_ARGUMENT;
  st = check_batch(rb, dims, false);
  if (st != MAMBA2_OK) return st;
  const int64_t Dc = (int64_t)dims->nheads * dims->headdim + 2 * (int64_t)dims->ngroups * dims->d_state;
  if (dims->conv_kernel < 2 || dims->conv_kernel > 4 || Dc % act_vec(dims->act_dtype) != 0)
    return MAMBA2_NOT_IMPLEMENTED;
  const int64_t n = snapshot_count(rb, snap_every);
  if (n > 0 && !conv_snaps) return MAMBA2_INVALID_ARGUMENT;
  if (n * (dims->conv_kernel - 1) >= kMaxElems) return MAMBA2_NOT_IMPLEMENTED;
  if (rb->num_rows == 0) return MAMBA2_OK;
  // the snapshots read the slot rows the conv then replaces: stream order keeps them first
  hipError_t e = launch_conv_snapshots(conv_snaps, x, conv_state, batch_dev(rb), snapshot_max_per_seq(rb, snap_every),
                                       (int32_t)Dc, dims->conv_kernel, snap_every, dims->act_dtype,
                                       (hipStream_t)stream);
  if (e != hipSuccess) return MAMBA2_HIP_ERROR;
  return from_hip(launch_conv1d(dst, x, weight, bias, conv_state, batch_dev(rb), (int32_t)Dc,
                                dims->conv_kernel, dims->act_dtype, (hipStream_t)stream));
}

size_t mamba2_scan_prefill_snap_workspace_bytes(const mamba2_recurrent_batch* rb, const mamba2_dims* dims,
                                                int32_t snap_every) {
  if (check_all(rb, dims, false) != MAMBA2_OK || rb->num_rows == 0) return 0;
  const int32_t L = scan_segment_length_snap(rb, dims, snap_every);
  return L > 0 ? scan_layout(rb, dims, L).total : 0;
}

mamba2_status mamba2_scan_prefill_snap(void* dst, const void* xbc, const void* dt, const float* a_log,
                                       const float* dt_bias, const float* d, float* ssm_state,
                                       float* ssm_snaps, int32_t snap_every,
                                       const mamba2_recurrent_batch* rb, const mamba2_dims* dims,
                                       void* workspace, size_t workspace_bytes, void* stream) {
  mamba2_status st = check_dims(dims);
  if (st != MAMBA2_OK) return st;
  if (!rb || snap_every < 1) return MAMBA2_INVALID_ARGUMENT;
  if (rb->num_rows > 0 && (!dst || !xbc || !dt || !a_log || !dt_bias || !d || !ssm_state))
    return MAMBA2_INVALID_ARGUMENT;
  if (!aligned16({dst, xbc, ssm_state, ssm_snaps})) return MAMBA2_INVALID_ARGUMENT;
  st = check_batch(rb, dims, false);
  if (st != MAMBA2_OK) return st;
  if (!scan_supported(dims)) return MAMBA2_NOT_IMPLEMENTED;
  const int32_t seg_len = scan_segment_length_snap(rb, dims, snap_every);
  if (seg_len == 0) return MAMBA2_NOT_IMPLEMENTED;
  const int64_t n = snapshot_count(rb, snap_every);
  if (n > 0 && !ssm_snaps) return MAMBA2_INVALID_ARGUMENT;
  if (n >= kMaxElems) return MAMBA2_NOT_IMPLEMENTED;
  if (rb->num_rows == 0) return MAMBA2_OK;
  const ScanLayout lay = scan_layout(rb, dims, seg_len);
  if (!workspace || workspace_bytes < lay.total) return MAMBA2_WORKSPACE_TOO_SMALL;
  if (((uintptr_t)workspace & 255) != 0) return MAMBA2_INVALID_ARGUMENT;
  // the snapshots are the states entering the segments that start at the boundaries: the MFMA
  // path's output kernel writes them as it obtains them; the generic path keeps every segment's
  // state and copies those afterwards
  if (scan_uses_mfma(dims)) {
    ScanArgs a{dst, xbc, dt, a_log, dt_bias, d, ssm_state, batch_dev(rb), *dims, lay, (char*)workspace, false,
               n > 0 ? ssm_snaps : nullptr, snap_every};
    return from_hip(launch_scan_prefill(a, (hipStream_t)stream));
  }
  ScanArgs a{dst, xbc, dt, a_log, dt_bias, d, ssm_state, batch_dev(rb), *dims, lay, (char*)workspace, true, nullptr, 0};
  hipError_t e = launch_scan_prefill(a, (hipStream_t)stream);
  if (e != hipSuccess) return MAMBA2_HIP_ERROR;
  return from_hip(launch_ssm_snapshots(a, ssm_snaps, snapshot_max_per_seq(rb, snap_every), snap_every,
                                       (hipStream_t)stream));
}

mamba2_status mamba2_scan_verify(void* dst, const void* xbc, const void* dt, const float* a_log,
                                 const float* dt_bias, const float* d, float* ssm_state, float* ssm_snaps,
                                 const mamba2_recurrent_batch* rb, const mamba2_dims* dims, void* stream) {
  mamba2_status st = check_dims(dims);
  if (st != MAMBA2_OK) return st;
  if (!rb) return MAMBA2_INVALID_ARGUMENT;
  if (rb->num_rows > 0 && (!dst || !xbc || !dt || !a_log || !dt_bias || !d || !ssm_state))
    return MAMBA2_INVALID_ARGUMENT;
  if (!aligned16({dst, xbc, ssm_state, ssm_snaps})) return MAMBA2_INVALID_ARGUMENT;
  st = check_batch(rb, dims, false);
  if (st != MAMBA2_OK) return st;
  int32_t max_rows = 0;
  for (int s = 0; s < rb->num_seqs; ++s) max_rows = std::max(max_rows, rb->run_lengths[s]);
  if (max_rows > kMaxVerifyRows) return MAMBA2_RUN_LENGTHS;
  if (!decode_supported(*dims) || !decode_grid_fits(*dims, rb->num_seqs)) return MAMBA2_NOT_IMPLEMENTED;
  if (verify_lds_bytes(*dims, kMaxVerifyRows) > 65536) return MAMBA2_NOT_IMPLEMENTED;
  if (rb->num_rows == 0) return MAMBA2_OK;
  return from_hip(launch_scan_verify(dst, xbc, dt, a_log, dt_bias, d, ssm_state, ssm_snaps, batch_dev(rb), *dims,
                                     max_rows, (hipStream_t)stream));
}

mamba2_status mamba2_commit_snapshots(float* ssm_state, void* conv_state, const float* ssm_snaps,
                                      const void* conv_snaps, int32_t snap_every, const int32_t* accepted,
                                      const mamba2_recurrent_batch* rb, const mamba2_dims* dims, void* stream) {
  mamba2_status st = check_dims(dims);
  if (st != MAMBA2_OK) return st;
  if (!rb || snap_every < 1) return MAMBA2_INVALID_ARGUMENT;
  if (rb->num_seqs > 0 && !accepted) return MAMBA2_INVALID_ARGUMENT;
  if ((ssm_snaps && !ssm_state) || (conv_snaps && !conv_state)) return MAMBA2_INVALID_ARGUMENT;
  if (!aligned16({ssm_state, conv_state, ssm_snaps, conv_snaps})) return MAMBA2_INVALID_ARGUMENT;
  st = check_batch(rb, dims, false);
  if (st != MAMBA2_OK) return st;
  const int64_t Dc = (int64_t)dims->nheads * dims->headdim + 2 * (int64_t)dims->ngroups * dims->d_state;
  if (dims->d_state % 4 != 0 || Dc % act_vec(dims->act_dtype) != 0 || dims->conv_kernel < 2)
    return MAMBA2_NOT_IMPLEMENTED;
  if (rb->num_seqs == 0 || (!ssm_snaps && !conv_snaps)) return MAMBA2_OK;
  return from_hip(launch_commit(ssm_state, conv_state, ssm_snaps, conv_snaps, accepted, batch_dev(rb), *dims,
                                snap_every, (hipStream_t)stream));
}

mamba2_status mamba2_padded_runs(const uint8_t* mask, int32_t batch, int32_t max_len, int32_t* run_lengths,
                                 int32_t* left_padded) {
  if (batch < 0 || max_len < 1 || (batch > 0 && (!mask || !run_lengths)) || !left_padded)
    return MAMBA2_INVALID_ARGUMENT;
  bool left_ok = true, right_ok = true;
  for (int b = 0; b < batch; ++b) {
    const uint8_t* m = mask + (size_t)b * max_len;
    int n = 0, first = -1, last = -1;
    for (int j = 0; j < max_len; ++j) {
      if (m[j]) {
        if (first < 0) first = j;
        last = j;
        ++n;
      }
    }
    if (n == 0 || last - first + 1 != n) return MAMBA2_INVALID_ARGUMENT;
    run_lengths[b] = n;
    left_ok = left_ok && last == max_len - 1;
    right_ok = right_ok && first == 0;
  }
  if (!left_ok && !right_ok) return MAMBA2_INVALID_ARGUMENT;
  *left_padded = left_ok && !right_ok ? 1 : 0;
  return MAMBA2_OK;
}


mamba2_status mamba2_pack_rows(void* dst, const void* src, int64_t row_bytes, int32_t max_len, int32_t left_padded,
                               const mamba2_recurrent_batch* rb, void* stream) {
  return padded_call(true, dst, src, row_bytes, max_len, left_padded, rb, stream);
}

mamba2_status mamba2_unpack_rows(void* dst, const void* src, int64_t row_bytes, int32_t max_len,
                                 int32_t left_padded, const mamba2_recurrent_batch* rb, void* stream) {
  return padded_call(false, dst, src, row_bytes, max_len, left_padded, rb, stream);
}

mamba2_status mamba2_linear(void* dst, const void* x, const void* weight, int64_t rows, int64_t out_features,
                            int64_t in_features, int32_t act_dtype, void* stream) {
  if (rows < 0 || out_features < 1 || in_features < 1) return MAMBA2_INVALID_ARGUMENT;
  if (act_dtype != MAMBA2_DTYPE_F32 && act_dtype != MAMBA2_DTYPE_BF16) return MAMBA2_INVALID_ARGUMENT;
  if (rows > 0 && (!dst || !x || !weight)) return MAMBA2_INVALID_ARGUMENT;
  if (!aligned16({dst, x, weight})) return MAMBA2_INVALID_ARGUMENT;
  if (rows == 0) return MAMBA2_OK;
  if (!linear_supported(rows, out_features, in_features, act_dtype)) return MAMBA2_NOT_IMPLEMENTED;
  return from_hip(launch_linear(dst, x, weight, rows, out_features, in_features, (hipStream_t)stream));
}

size_t mamba2_ssm_slot_bytes(const mamba2_dims* d) {
  if (check_dims(d) != MAMBA2_OK) return 0;
  return (size_t)d->nheads * d->headdim * d->d_state * sizeof(float);
}

size_t mamba2_conv_slot_bytes(const mamba2_dims* d) {
  if (check_dims(d) != MAMBA2_OK) return 0;
  const size_t Dc = (size_t)d->nheads * d->headdim + 2 * (size_t)d->ngroups * d->d_state;
  return (size_t)(d->conv_kernel - 1) * Dc * (d->act_dtype == MAMBA2_DTYPE_BF16 ? 2 : 4);
}

const char* mamba2_status_string(mamba2_status s) {
  switch (s) {
    case MAMBA2_OK: return "ok";
    case MAMBA2_INVALID_ARGUMENT: return "invalid argument";
    case MAMBA2_SLOT_OUT_OF_RANGE: return "slot out of range";
    case MAMBA2_SLOT_SHARED: return "slot shared by two sequences";
    case MAMBA2_RUN_LENGTHS: return "run lengths do not cover the rows";
    case MAMBA2_WORKSPACE_TOO_SMALL: return "workspace too small";
    case MAMBA2_NOT_IMPLEMENTED: return "not implemented for these dims";
    case MAMBA2_HIP_ERROR: return "HIP error";
  }
  return "unknown status";
}

}  // extern "C"
