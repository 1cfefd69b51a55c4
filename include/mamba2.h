/*
 * mamba2.h - C ABI of the Mamba2 mixer hot path on AMD Instinct MI355X (gfx950).
 *
 * The path, as the page "feat(backend): Mamba2 ops, with CPU reference
 * implementations" (gllm PR #85) defines it in its section "Ops":
 *
 *   1. CausalConv1D: a depthwise causal conv over each sequence's run of rows,
 *      fused with SiLU, preceded by the sequence's last kernel-1 inputs from its
 *      conv-state slot (zeros when fresh); the slot then holds the last kernel-1
 *      inputs.                                             -> mamba2_conv1d
 *   2. SSMScan: dt' = softplus(dt + dt_bias) (no clamp), per token
 *      h = h * exp(-exp(A_log) * dt') + dt' * B (x) x and y = h . C + D * x, head h
 *      reading B and C of group h / (heads / groups), the state seeded from and
 *      written back to the sequence's SSM slot.     -> mamba2_scan_prefill (a
 *      chunked parallel scan over packed variable-length runs) and
 *      mamba2_scan_decode (one row per sequence).
 *   3. GatedRMSNorm: rmsnorm(x * silu(z)) * weight, the RMS taken per group.
 *                                                      -> mamba2_gated_rmsnorm
 *
 * The stateful calls take a mamba2_recurrent_batch: per sequence its run length,
 * slot and fresh flag (same page, section "Ops": a fresh sequence starts from
 * zero and never reads its slot; a slot out of range, a slot shared by two
 * sequences and run lengths that do not cover the rows are rejected).
 *
 * Conventions for every call
 *   - Memory: the caller allocates every buffer; the library keeps no pointer
 *     past the call and allocates no device memory.  "device" pointers are HIP
 *     device memory; "host" pointers are read during the call only.
 *   - Layout: row-major, last index contiguous.  An xBC row is
 *     [x (H*P, head h at h*P+p) | B (G*N, group g at g*N+n) | C (G*N)],
 *     Dc = H*P + 2*G*N channels; Di = H*P.
 *   - Alignment: dst, x/xbc, z, the state pools and the conv/norm weight and
 *     bias vectors must be 16-byte aligned (the kernels move them in 16-byte
 *     units), else MAMBA2_INVALID_ARGUMENT; dt, a_log, dt_bias and d need only
 *     their element alignment.
 *   - Types: activations, conv state and outputs in the activation type
 *     (MAMBA2_DTYPE_F32 or MAMBA2_DTYPE_BF16; bf16 as its 16 raw bits); SSM
 *     state, weights, biases, A_log, dt_bias and D are fp32.
 *   - Mutation: only the output and the named state slots are written; inputs
 *     are never written; the output must not alias any input; slots not named by
 *     the batch are left bit-identical.
 *   - Errors: every check runs on the host before the first launch.  On error
 *     nothing is enqueued and nothing is written.  No call throws.
 *   - Streams: calls only enqueue on `stream` (a hipStream_t; NULL is the null
 *     stream) and return; no host synchronisation, no allocation, no copy.
 *     Device buffers must stay valid until the stream work completes.
 */
#ifndef MAMBA2_H
#define MAMBA2_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum mamba2_status {
  MAMBA2_OK = 0,
  MAMBA2_INVALID_ARGUMENT = 1,   /* null pointer, bad dims or dtype, bad groups/eps */
  MAMBA2_SLOT_OUT_OF_RANGE = 2,  /* a slot < 0 or >= pool_slots */
  MAMBA2_SLOT_SHARED = 3,        /* two sequences of one batch name the same slot */
  MAMBA2_RUN_LENGTHS = 4,        /* a length <= 0, sum != num_rows, or decode length != 1 */
  MAMBA2_WORKSPACE_TOO_SMALL = 5,
  MAMBA2_NOT_IMPLEMENTED = 6,    /* valid dims the kernels do not cover */
  MAMBA2_HIP_ERROR = 7           /* the runtime reported a launch failure */
} mamba2_status;

typedef enum mamba2_dtype { MAMBA2_DTYPE_F32 = 0, MAMBA2_DTYPE_BF16 = 1 } mamba2_dtype;

/* Sizes of one mixer layer. */
typedef struct mamba2_dims {
  int32_t nheads;      /* H >= 1 */
  int32_t headdim;     /* P >= 1 */
  int32_t d_state;     /* N >= 1 */
  int32_t ngroups;     /* G >= 1, H % G == 0 */
  int32_t conv_kernel; /* K, 2..4; the conv state holds K-1 rows */
  int32_t chunk_size;  /* Q >= 1: chunk length of the chunked scan (see mamba2_scan_prefill) */
  int32_t pool_slots;  /* M >= 0: slots in each state pool */
  int32_t act_dtype;   /* mamba2_dtype of activations, outputs and conv state */
} mamba2_dims;

/*
 * One batch of sequences, packed row after row in cu_seqlens order.
 * The host arrays are validated; the device arrays are what the kernels read
 * and must hold the same values (dev_cu_seqlens[s] = sum of run_lengths[0..s),
 * dev_cu_seqlens[S] = num_rows).  The library does not read device arrays on
 * the host, so a mismatch between the two copies is the caller's error.
 */
typedef struct mamba2_recurrent_batch {
  int32_t num_seqs;               /* S >= 0 */
  int32_t num_rows;               /* T = sum of run_lengths */
  const int32_t* run_lengths;     /* host   [S], each >= 1 */
  const int32_t* slots;           /* host   [S], distinct, in [0, pool_slots) */
  const uint8_t* fresh;           /* host   [S], nonzero: start from zero, never read the slot */
  const int32_t* dev_cu_seqlens;  /* device [S+1] */
  const int32_t* dev_slots;       /* device [S] */
  const uint8_t* dev_fresh;       /* device [S] */
} mamba2_recurrent_batch;

/*
 * Depthwise causal conv1d fused with SiLU, with per-sequence conv-state slots
 * (gllm PR #85, "Ops", CausalConv1D):
 *   dst[r, c] = silu(bias[c] + sum_{k=0}^{K-1} weight[c, k] * win[t + k]),
 * where row r is row t of its sequence and win is the sequence's history (K-1
 * rows from conv_state[slot], or zeros when fresh) followed by its rows of x;
 * weight[c, K-1] multiplies the current row.  Afterwards conv_state[slot] holds
 * the last K-1 rows of win, copied bit for bit.
 *   dst        device [T, Dc] act (written)
 *   x          device [T, Dc] act, the xBC rows before the conv
 *   weight     device [Dc, K] f32;  bias device [Dc] f32
 *   conv_state device [M, K-1, Dc] act, row 0 the oldest (slots of rb read/written)
 * Needs Dc % 8 == 0 (bf16) or Dc % 4 == 0 (f32), else MAMBA2_NOT_IMPLEMENTED.
 */
mamba2_status mamba2_conv1d(void* dst, const void* x, const float* weight, const float* bias,
                            void* conv_state, const mamba2_recurrent_batch* rb,
                            const mamba2_dims* dims, void* stream);

/*
 * Selective scan over packed variable-length prefill runs (gllm PR #85, "Ops",
 * SSMScan), computed as a chunked parallel scan: within a chunk the outputs
 * come from the quadratic (masked C.B^T) form, across chunks from the carried
 * state.  In exact arithmetic this equals the per-token recurrence, so the
 * results do not depend on the chunk length (dims->chunk_size sets the chunk of
 * the fp32 path; the bf16 MFMA path for P = 64, N = 128 uses 64-row chunks).
 *   dst       device [T, Di] act (y, written)
 *   xbc       device [T, Dc] act, the conv output; x, B, C at fixed offsets
 *   dt        device [T, H] act;  a_log, dt_bias, d: device [H] f32
 *   ssm_state device [M, H, P, N] f32: seeded from (unless fresh) and written to
 *             the slot of every sequence
 *   workspace device, >= mamba2_scan_prefill_workspace_bytes(rb, dims) bytes,
 *             256-byte aligned; contents on entry are ignored.
 */
mamba2_status mamba2_scan_prefill(void* dst, const void* xbc, const void* dt, const float* a_log,
                                  const float* dt_bias, const float* d, float* ssm_state,
                                  const mamba2_recurrent_batch* rb, const mamba2_dims* dims,
                                  void* workspace, size_t workspace_bytes, void* stream);

/* Workspace bytes mamba2_scan_prefill needs for this batch (0 when S == 0). */
size_t mamba2_scan_prefill_workspace_bytes(const mamba2_recurrent_batch* rb,
                                           const mamba2_dims* dims);

/*
 * mamba2_scan_prefill for callers that cannot allocate device memory (code under HIP
 * graph capture, tight serving loops, harnesses that forbid allocation): the same scan,
 * with no workspace argument.  Its workspace is a fixed 32 MiB array of the library's
 * own, one per GPU, held until the process ends (looked up on the first call on each
 * device); the call allocates nothing.  When the usual segment length's workspace does
 * not fit, longer segments are used (bf16 P = 64, N = 128 path: up to 4096 rows), which
 * can change results within rounding; a batch whose workspace does not fit even then
 * is rejected with MAMBA2_WORKSPACE_TOO_SMALL before any launch (e.g. 48 heads x 64 x 128
 * fits up to ~20 segments of 4096 rows).  Every call on a GPU shares that GPU's array:
 * calls that overlap in time on one GPU (two streams, two threads) race.  Arguments,
 * requirements and other errors as mamba2_scan_prefill.
 */
mamba2_status mamba2_scan_prefill_static(void* dst, const void* xbc, const void* dt, const float* a_log,
                                         const float* dt_bias, const float* d, float* ssm_state,
                                         const mamba2_recurrent_batch* rb, const mamba2_dims* dims, void* stream);

/*
 * One-row decode step of the same recurrence (every run length must be 1):
 * each sequence's fp32 state is read once from its slot (not at all when fresh)
 * and written back once.  Arguments as mamba2_scan_prefill, no workspace.
 * Needs d_state % 4 == 0 with d_state / 4 a power of two <= 64, and
 * headdim * d_state / 4 a multiple of 512, equal to 256, or below 256 and a
 * multiple of 64 (whole 64-lane wavefronts), else MAMBA2_NOT_IMPLEMENTED.
 */
mamba2_status mamba2_scan_decode(void* dst, const void* xbc, const void* dt, const float* a_log,
                                 const float* dt_bias, const float* d, float* ssm_state,
                                 const mamba2_recurrent_batch* rb, const mamba2_dims* dims,
                                 void* stream);

/*
 * Gated RMSNorm (gllm PR #85, "Ops", GatedRMSNorm; the gate is applied before
 * the norm): for each row and each of `groups` column groups of size
 * d_inner / groups,
 *   g = x * silu(z),  dst = g / sqrt(mean_group(g^2) + eps) * weight.
 *   dst, x, z device [rows, d_inner] act;  weight device [d_inner] f32.
 * Needs (d_inner / groups) % 8 == 0 (bf16) or % 4 == 0 (f32), else
 * MAMBA2_NOT_IMPLEMENTED; groups must divide d_inner; eps >= 0 and finite.
 */
mamba2_status mamba2_gated_rmsnorm(void* dst, const void* x, const void* z, const float* weight,
                                   int32_t groups, float eps, int32_t rows, int32_t d_inner,
                                   int32_t act_dtype, void* stream);

/*
 * State snapshots and rollback.  "feat(mamba2): integrate model loading and
 * recurrent inference" (InfiniLM PR #575), section "Notes for Reviewers", names
 * prefix-state snapshots and speculative rollback as variants that adaptation
 * leaves out; the calls below provide them.  A snapshot at boundary b of a
 * sequence is the state that a run of only its first b rows would leave in its
 * slots: the SSM state [H, P, N] f32 after row b, and the conv state [K-1, Dc]
 * act (the last K-1 entries of history ++ rows[0, b)).  With a stride
 * snap_every = E >= 1 the boundaries are E, 2E, ... strictly inside each run
 * (b < L; the state after the whole run is in the slots).  Snapshots are packed
 * sequence after sequence in batch order: sequence s owns floor((L_s - 1) / E)
 * of them, boundary j E at index first(s) + j - 1, first(s) the count owned by
 * the sequences before it.  A snapshot has the layout of one pool slot, so the
 * snapshot buffers may be free slots of the caller's own pools (the snapshot
 * pointers set to slot `base` of each pool): rolling a sequence back is then a
 * change of its slot number, with no copy; mamba2_commit_snapshots is the
 * copying alternative.
 */

/* Snapshots a batch holds at stride snap_every (host only); -1 on a null batch,
 * a run length < 1 or snap_every < 1. */
int64_t mamba2_snapshot_count(const mamba2_recurrent_batch* rb, int32_t snap_every);

/*
 * mamba2_conv1d plus its conv-state snapshots every snap_every rows.
 *   conv_snaps device [count, K-1, Dc] act (written; may be NULL when count is 0)
 * Other arguments, requirements and errors as mamba2_conv1d.
 */
mamba2_status mamba2_conv1d_snap(void* dst, const void* x, const float* weight, const float* bias,
                                 void* conv_state, void* conv_snaps, int32_t snap_every,
                                 const mamba2_recurrent_batch* rb, const mamba2_dims* dims, void* stream);

/*
 * mamba2_scan_prefill plus SSM-state snapshots every snap_every rows (prefix
 * caching).  The chunked scan then cuts its segments so that every boundary
 * starts one, and copies the states entering those segments.
 *   ssm_snaps device [count, H, P, N] f32 (written; may be NULL when count is 0)
 *   workspace >= mamba2_scan_prefill_snap_workspace_bytes(rb, dims, snap_every)
 * snap_every must be a multiple of 64 on the bf16 P = 64, N = 128 path and of
 * min(chunk_size, 64) on the other, else MAMBA2_NOT_IMPLEMENTED.  Other
 * arguments, requirements and errors as mamba2_scan_prefill.
 */
mamba2_status mamba2_scan_prefill_snap(void* dst, const void* xbc, const void* dt, const float* a_log,
                                       const float* dt_bias, const float* d, float* ssm_state,
                                       float* ssm_snaps, int32_t snap_every,
                                       const mamba2_recurrent_batch* rb, const mamba2_dims* dims,
                                       void* workspace, size_t workspace_bytes, void* stream);

/* Workspace bytes mamba2_scan_prefill_snap needs (0 when S == 0 or snap_every
 * is not supported). */
size_t mamba2_scan_prefill_snap_workspace_bytes(const mamba2_recurrent_batch* rb,
                                                const mamba2_dims* dims, int32_t snap_every);

/*
 * A short run per sequence, e.g. the draft tokens of speculative decoding to be
 * verified: runs of 1..16 rows (MAMBA2_RUN_LENGTHS beyond), the recurrence applied
 * row after row in the decode mapping (each sequence's state is read once and
 * written once; a run of one row gives mamba2_scan_decode's results bit for bit).
 *   ssm_snaps device [T - S, H, P, N] f32: the state after every row but the last
 *             (snap_every = 1 snapshots), or NULL to skip them
 * Other arguments as mamba2_scan_decode; the shapes it covers, else
 * MAMBA2_NOT_IMPLEMENTED.
 */
mamba2_status mamba2_scan_verify(void* dst, const void* xbc, const void* dt, const float* a_log,
                                 const float* dt_bias, const float* d, float* ssm_state, float* ssm_snaps,
                                 const mamba2_recurrent_batch* rb, const mamba2_dims* dims, void* stream);

/*
 * Rollback to the accepted prefix of each run: sequence s accepted its first
 * m = accepted[s] rows; when 1 <= m < L_s and m % snap_every == 0 its slots take
 * the snapshots at boundary m; otherwise (m == L_s: the slots already hold the
 * whole run's state; any other value) they are left as they are.  rb and
 * snap_every are those of the run that made the snapshots.
 *   ssm_state, ssm_snaps:  device, as above (ssm_snaps NULL: the SSM pool is not touched)
 *   conv_state, conv_snaps: device, as above (conv_snaps NULL: the conv pool is not touched)
 *   accepted  device [S] int32
 */
mamba2_status mamba2_commit_snapshots(float* ssm_state, void* conv_state, const float* ssm_snaps,
                                      const void* conv_snaps, int32_t snap_every, const int32_t* accepted,
                                      const mamba2_recurrent_batch* rb, const mamba2_dims* dims, void* stream);

/*
 * The projections around the path (a linear layer; the layer of "Granite Mamba2
 * Inference Optimization" maps its hidden states to z, xBC and dt before the
 * conv and the norm's output back to the model width after it):
 *   dst[m, n] = sum_k x[m, k] * weight[n, k]   (fp32 accumulation, one rounding)
 *   dst    device [rows, out_features] act (written; must not alias x or weight)
 *   x      device [rows, in_features] act
 *   weight device [out_features, in_features] act, one row per output feature
 * A row slice of a weight is itself a weight, so in_proj is one call per output
 * part (z, xBC, dt) on the matching rows of its weight, each writing its own
 * contiguous tensor.  dst, x and weight 16-byte aligned, else
 * MAMBA2_INVALID_ARGUMENT.  Covers bf16 with out_features and in_features multiples
 * of 8 (and rows * in_features, rows * out_features, out_features * in_features
 * below 2^31), else MAMBA2_NOT_IMPLEMENTED.
 */
mamba2_status mamba2_linear(void* dst, const void* x, const void* weight, int64_t rows, int64_t out_features,
                            int64_t in_features, int32_t act_dtype, void* stream);

/*
 * Padded batches.  The layer entry of "Granite Mamba2 Inference Optimization"
 * takes hidden states [B, Lmax] with an attention mask and must match across
 * variable-length padded batches.  Reading: the real rows of each batch row form
 * one run, at the end of every row (left padding) or at the start of every row
 * (right padding); that run is the row's sequence and the padding rows are not
 * part of it.  The caller builds a RecurrentBatch from the run lengths (its slot
 * and fresh flag per batch row, fresh = no previous state), packs the padded
 * inputs, runs the path and unpacks the output.
 */

/* Host only: run lengths [batch] and the padding side (1 left, 0 right; a batch
 * without padding reports 0) of a host mask [batch, max_len] (nonzero = real).
 * MAMBA2_INVALID_ARGUMENT for a row without real rows, a gap inside a run, or
 * runs on both sides. */
mamba2_status mamba2_padded_runs(const uint8_t* mask, int32_t batch, int32_t max_len, int32_t* run_lengths,
                                 int32_t* left_padded);

/*
 * dst [T, row] <- the real rows of src [S, max_len, row], batch row after batch
 * row (pack), or dst [S, max_len, row] <- the packed rows at their padded
 * positions with zero bytes on the padding (unpack).  Rows are copied as
 * row_bytes bytes (any element type).  rb: the batch built from the run
 * lengths (its slots and fresh flags are not used here); each run length must be
 * at most max_len, else MAMBA2_RUN_LENGTHS.  device buffers; no alignment needed
 * (the copy unit adapts to the row size and the pointers).
 */
mamba2_status mamba2_pack_rows(void* dst, const void* src, int64_t row_bytes, int32_t max_len, int32_t left_padded,
                               const mamba2_recurrent_batch* rb, void* stream);
mamba2_status mamba2_unpack_rows(void* dst, const void* src, int64_t row_bytes, int32_t max_len,
                                 int32_t left_padded, const mamba2_recurrent_batch* rb, void* stream);

/*
 * Host-only checks shared by every stateful call (no device access):
 * dims, then run lengths (each >= 1; decode != 0: each == 1; sum == num_rows),
 * then slot range, then slot sharing.  Returns the first failing status.
 */
mamba2_status mamba2_validate(const mamba2_recurrent_batch* rb, const mamba2_dims* dims,
                              int32_t decode);

/*
 * Bytes of one slot: fp32 SSM state H*P*N*4, conv state (K-1)*Dc*sizeof(act).
 * ("feat(mamba2): integrate model loading and recurrent inference", InfiniLM
 * PR #575, section "Motivation": conv plus FP32 SSM state per request, constant
 * in the history length.)
 */
size_t mamba2_ssm_slot_bytes(const mamba2_dims* dims);
size_t mamba2_conv_slot_bytes(const mamba2_dims* dims);

const char* mamba2_status_string(mamba2_status status);

/*
 * Kernel timing.  While enabled, the library records a pair of HIP events on the
 * launch stream around every kernel it launches (creating the events costs
 * nothing at launch time: a pool of `capacity` pairs is made by the enable
 * call).  mamba2_timing_collect waits for the recorded events, writes up to
 * `max` records, resets the log and returns how many it wrote (< 0 on error).
 * Not thread-safe; meant for benchmarks.
 */
typedef struct mamba2_kernel_time {
  const char* name; /* static string: the kernel's name */
  float ms;         /* duration between the two events */
} mamba2_kernel_time;

mamba2_status mamba2_timing_enable(int32_t capacity); /* capacity 0 disables */
int32_t mamba2_timing_collect(mamba2_kernel_time* out, int32_t max);

#ifdef __cplusplus
}
#endif

#endif /* MAMBA2_H */
