/*
 * mamba3.h - C ABI of the Mamba-3 SISO forward over packed variable-length sequences,
 * on AMD Instinct MI355X (gfx950), in the same library as mamba2.h.
 *
 * The operator of "Mamba-3 SISO Long-Ragged Multi-Chunk Joint States Full VJP", section
 * "What You Have" (steps 1-7) and section "Hard Constraints" (dtypes).  Per packed
 * sequence (cu_seqlens; everything resets at each boundary) and value head h:
 *   - one Q/K head shared by the H value heads;
 *   - theta = tanh(angles) * pi; the rotary angle of token t is the running sum over the
 *     sequence of theta * dt[., h], mod 2 pi (angles [T, NA] shared by the heads);
 *   - q + q_bias[h], k + k_bias[h], then paired rotary: pair a < NA is components
 *     (2a, 2a + 1), turned by the angle of pair a; components from 2 NA on unrotated;
 *   - p = sigmoid(trap); shifted_gamma_t = dt_{t+1} (1 - p_{t+1}) (0 at the sequence's last
 *     token); scale_t = dt_t p_t + shifted_gamma_t;
 *   - y_t = sum_{s<=t} exp(sum_{r=s+1..t} adt_r) (qh_t . kh_s) scale_s v_s + d[h] v_t
 *           - shifted_gamma_t (qh_t . kh_t) v_t  (adt: the per-token log of the decay);
 *   - out_t = y_t * z_t * sigmoid(z_t);
 *   - final states per sequence: the last token's rotary angle, the SSM state
 *     sum_s exp(sum_{r>s} adt_r) scale_s v_s kh_s^T, the last token's rotated key and value.
 *
 * Conventions as mamba2.h: caller-owned memory, checks before any launch (nothing enqueued
 * on error), stream-ordered and asynchronous, status codes of mamba2_status, bf16 as raw
 * 16-bit words.  Inputs are never written.
 */
#ifndef MAMBA3_H
#define MAMBA3_H

#include <stddef.h>
#include <stdint.h>

#include "mamba2.h"

#ifdef __cplusplus
extern "C" {
#endif

typedef struct mamba3_dims {
  int32_t nheads;  /* H value heads (one shared Q/K head) */
  int32_t qk_dim;  /* DK: query / key width */
  int32_t v_dim;   /* DV: value width */
  int32_t nangles; /* NA rotary pairs, 2 NA <= DK */
} mamba3_dims;

typedef struct mamba3_varlen {
  int32_t num_seqs;              /* S >= 0 */
  int32_t num_rows;              /* T = sum of run_lengths */
  const int32_t* run_lengths;    /* host [S], each >= 1 */
  const int32_t* dev_cu_seqlens; /* device [S + 1], the exclusive prefix sums of run_lengths */
} mamba3_varlen;

/*
 * The forward, chunked over 64-row chunks (each within one sequence).
 *   out          device [T, H, DV] bf16 (written)
 *   final_angle  device [S, H, NA] bf16; final_ssm [S, H, DV, DK] f32;
 *   final_k      device [S, H, DK] f32;  final_v [S, H, DV] bf16 (written)
 *   q, k         device [T, DK] bf16;  v, z [T, H, DV] bf16;  trap [T, H] bf16;
 *   angles       device [T, NA] bf16 (final_angle and angles may be NULL when NA = 0)
 *   adt, dt      device [T, H] f32;  q_bias, k_bias [H, DK] f32;  d [H] f32
 *   workspace    device, >= mamba3_siso_forward_workspace_bytes(batch, dims) bytes,
 *                256-byte aligned; contents on entry ignored.
 * out, final_ssm, final_k, q, k, v, z, q_bias, k_bias 16-byte aligned, else
 * MAMBA2_INVALID_ARGUMENT.  Covers DK a multiple of 16 up to 128, DV a multiple of 16 up to 64,
 * NA up to 64, else MAMBA2_NOT_IMPLEMENTED; a run length < 1 or a sum other than num_rows:
 * MAMBA2_RUN_LENGTHS.
 */
mamba2_status mamba3_siso_forward(void* out, void* final_angle, float* final_ssm, float* final_k, void* final_v,
                                  const void* q, const void* k, const void* v, const float* adt, const float* dt,
                                  const void* trap, const float* q_bias, const float* k_bias, const void* angles,
                                  const float* d, const void* z, const mamba3_varlen* batch, const mamba3_dims* dims,
                                  void* workspace, size_t workspace_bytes, void* stream);

/* Workspace bytes mamba3_siso_forward needs (0 when T == 0 or the arguments are rejected). */
size_t mamba3_siso_forward_workspace_bytes(const mamba3_varlen* batch, const mamba3_dims* dims);

#ifdef __cplusplus
}
#endif

#endif /* MAMBA3_H */
