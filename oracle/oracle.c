/*
 * Plain CPU oracle for the Mamba2 mixer hot path.
 *
 * TEST INFRASTRUCTURE ONLY.  Only the tests, the smoke check and the bench's
 * CPU-baseline leg may load this library.  It shares no code, header, table or
 * helper with the GPU library: it is written from the definitions on the pages,
 * one operation at a time, in scalar loops, so that a reader can check it
 * against them by eye.
 *
 * Sources (page title -> section):
 *   [gllm#85]  "feat(backend): Mamba2 ops, with CPU reference implementations",
 *              sections "Ops" (CausalConv1D, SSMScan, GatedRMSNorm, the
 *              RecurrentBatch rule), "CPU reference" (per-token recurrence, F32
 *              state rounding) and "Testing" (worked examples).
 *   [InfiniLM#575] "feat(mamba2): integrate model loading and recurrent
 *              inference", section "Motivation" (conv + FP32 SSM state per
 *              request) and "Notes for Reviewers" (head-wise D, gated RMSNorm
 *              after gating, unbounded time steps; prefix-state snapshots and
 *              speculative rollback named as variants that adaptation leaves
 *              out, which the snapshot functions below provide).
 *
 * Arithmetic: every operation is carried out in double from values widened
 * from their stored type.  Results are rounded once to the activation type
 * (fp32, or fp32 then bf16, both round-to-nearest-even).  The SSM state is
 * rounded to fp32 after every token, as [gllm#85] "CPU reference" states.
 *
 * Parallelism: OpenMP over independent units only ((sequence, channel) for the
 * conv, (sequence, head) for the scan, rows for the norm), so results do not
 * depend on the thread count.
 *
 * Build: gcc -O2 -ffp-contract=off -fopenmp -shared -fPIC oracle.c -lm
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

/* Status numbering of the C ABI (same numbers, defined here independently). */
enum {
  ORC_OK = 0,
  ORC_INVALID_ARGUMENT = 1,
  ORC_SLOT_OUT_OF_RANGE = 2,
  ORC_SLOT_SHARED = 3,
  ORC_RUN_LENGTHS = 4,
};

enum { ORC_F32 = 0, ORC_BF16 = 1 };

/* ---------------------------------------------------------------- storage */

static double bf16_bits_to_double(uint16_t b) {
  uint32_t u = (uint32_t)b << 16;
  float f;
  memcpy(&f, &u, 4);
  return (double)f;
}

/* float -> bf16, round to nearest, ties to even; NaN stays NaN. */
static uint16_t float_to_bf16_rne(float f) {
  uint32_t u;
  memcpy(&u, &f, 4);
  if ((u & 0x7fffffffu) > 0x7f800000u) return (uint16_t)((u >> 16) | 0x0040u);
  uint32_t lsb = (u >> 16) & 1u;
  u += 0x7fffu + lsb;
  return (uint16_t)(u >> 16);
}

static double load_act(const void* base, size_t i, int act) {
  if (act == ORC_F32) return (double)((const float*)base)[i];
  return bf16_bits_to_double(((const uint16_t*)base)[i]);
}

/* Round a double result once to the activation type and store it. */
static void store_act(void* base, size_t i, int act, double v) {
  float f = (float)v; /* double -> float, round to nearest even */
  if (act == ORC_F32)
    ((float*)base)[i] = f;
  else
    ((uint16_t*)base)[i] = float_to_bf16_rne(f);
}

static size_t act_size(int act) { return act == ORC_F32 ? 4 : 2; }

/* ------------------------------------------------------------ validation */

/*
 * The RecurrentBatch rules of [gllm#85] "Ops": a slot out of range, a slot
 * shared by two sequences of one batch, and run lengths that do not cover the
 * rows are rejected before anything is written.  Checked in this order:
 * run lengths (each >= 1, decode: each == 1, sum == rows), slot range, sharing.
 */
static int check_batch(int S, int T, const int32_t* len, const int32_t* slot, int M, int decode) {
  if (S < 0 || T < 0 || M < 0) return ORC_INVALID_ARGUMENT;
  if (S > 0 && (len == NULL || slot == NULL)) return ORC_INVALID_ARGUMENT;
  long long sum = 0;
  for (int s = 0; s < S; ++s) {
    if (len[s] <= 0) return ORC_RUN_LENGTHS;
    if (decode && len[s] != 1) return ORC_RUN_LENGTHS;
    sum += len[s];
  }
  if (sum != T) return ORC_RUN_LENGTHS;
  for (int s = 0; s < S; ++s)
    if (slot[s] < 0 || slot[s] >= M) return ORC_SLOT_OUT_OF_RANGE;
  for (int s = 0; s < S; ++s)
    for (int t = s + 1; t < S; ++t)
      if (slot[s] == slot[t]) return ORC_SLOT_SHARED;
  return ORC_OK;
}

int oracle_check_batch(int S, int T, const int32_t* len, const int32_t* slot, int M, int decode) {
  return check_batch(S, T, len, slot, M, decode);
}

static void first_rows(int S, const int32_t* len, long long* r0) {
  long long r = 0;
  for (int s = 0; s < S; ++s) {
    r0[s] = r;
    r += len[s];
  }
}

/* --------------------------------------------------------------- snapshots */

/*
 * State snapshots.  A snapshot at boundary b of a sequence is the state that a
 * run of only its first b rows would leave in the slot: for the SSM the state
 * after row b (the recurrence's h), for the conv the last K-1 entries of
 * history ++ rows[0, b).  With a stride E >= 1 the boundaries are b = E, 2E, ...
 * strictly inside the run (b < L; the state after the whole run is the slot).
 * Snapshots are packed sequence after sequence in batch order; sequence s owns
 * floor((L_s - 1) / E) of them, boundary j E at index first[s] + j - 1.
 */
static void snap_first(int S, const int32_t* len, int E, long long* first) {
  long long n = 0;
  for (int s = 0; s < S; ++s) {
    first[s] = n;
    n += (len[s] - 1) / E;
  }
}

long long oracle_snapshot_count(int S, const int32_t* len, int E) {
  if (S < 0 || E < 1) return -1;
  long long n = 0;
  for (int s = 0; s < S; ++s) {
    if (len[s] < 1) return -1;
    n += (len[s] - 1) / E;
  }
  return n;
}

/* ------------------------------------------------------------------ conv */

/*
 * CausalConv1D, [gllm#85] "Ops": for each sequence, the run of rows is preceded
 * by the K-1 inputs held in the sequence's conv-state slot (zeros when fresh;
 * a fresh sequence never reads its slot).  Output row t of channel c is
 *   silu(bias[c] + sum_{k=0}^{K-1} w[c][k] * win[t + k]),
 * win = history ++ rows, so w[c][K-1] multiplies the current row (the worked
 * example in "Testing" fixes this).  Afterwards the slot holds the last K-1
 * entries of win, copied bit for bit (older history shifts up when the run is
 * shorter than K-1).
 *
 * Layouts: x, dst [T][Dc] act; w [Dc][K] f32; b [Dc] f32;
 *          conv_state [M][K-1][Dc] act, row 0 the oldest.
 */
static int conv_impl(void* dst, const void* x, const float* w, const float* b, void* conv_state,
                     int S, int T, const int32_t* len, const int32_t* slot, const uint8_t* fresh,
                     int Dc, int K, int M, int act, void* snaps, int E) {
  if (Dc <= 0 || K < 1 || (act != ORC_F32 && act != ORC_BF16)) return ORC_INVALID_ARGUMENT;
  if (snaps != NULL && E < 1) return ORC_INVALID_ARGUMENT;
  int st = check_batch(S, T, len, slot, M, 0);
  if (st != ORC_OK) return st;
  if (S == 0) return ORC_OK;
  if (fresh == NULL) return ORC_INVALID_ARGUMENT;
  long long* r0 = (long long*)malloc(sizeof(long long) * (size_t)S);
  first_rows(S, len, r0);
  long long* sf = (long long*)malloc(sizeof(long long) * (size_t)S);
  if (snaps != NULL) snap_first(S, len, E, sf);
  const size_t es = act_size(act);
  const int H1 = K - 1;

#pragma omp parallel for collapse(2) schedule(dynamic, 16)
  for (int s = 0; s < S; ++s) {
    for (int c = 0; c < Dc; ++c) {
      const int L = len[s];
      unsigned char* slot_base = (unsigned char*)conv_state + (size_t)slot[s] * (size_t)H1 * Dc * es;
      const unsigned char* xb = (const unsigned char*)x;
      /* history as raw bits (so the new state is an exact copy) */
      unsigned char hist[16 * 4];
      unsigned char* hb = H1 <= 16 ? hist : (unsigned char*)malloc((size_t)H1 * es);
      for (int r = 0; r < H1; ++r) {
        if (fresh[s])
          memset(hb + (size_t)r * es, 0, es);
        else
          memcpy(hb + (size_t)r * es, slot_base + ((size_t)r * Dc + c) * es, es);
      }
      for (int t = 0; t < L; ++t) {
        double pre = (double)b[c];
        for (int k = 0; k < K; ++k) {
          int idx = t + k; /* position in win */
          double v;
          if (idx < H1) {
            v = load_act(hb, (size_t)idx, act);
          } else {
            v = load_act(x, (size_t)(r0[s] + idx - H1) * Dc + c, act);
          }
          pre += (double)w[(size_t)c * K + k] * v;
        }
        double out = pre / (1.0 + exp(-pre));
        store_act(dst, (size_t)(r0[s] + t) * Dc + c, act, out);
      }
      /* snapshots: at boundary bd the last K-1 entries of win[0, H1 + bd) */
      if (snaps != NULL) {
        for (int j = 1; (long long)j * E < L; ++j) {
          const int bd = j * E;
          unsigned char* sb = (unsigned char*)snaps + (size_t)(sf[s] + j - 1) * (size_t)H1 * Dc * es;
          for (int r = 0; r < H1; ++r) {
            int idx = bd + r;
            const unsigned char* src;
            if (idx < H1)
              src = hb + (size_t)idx * es;
            else
              src = xb + ((size_t)(r0[s] + idx - H1) * Dc + c) * es;
            memcpy(sb + ((size_t)r * Dc + c) * es, src, es);
          }
        }
      }
      /* new state: the last K-1 entries of win (win has H1 + L entries) */
      for (int r = 0; r < H1; ++r) {
        int idx = L + r;
        const unsigned char* src;
        if (idx < H1)
          src = hb + (size_t)idx * es;
        else
          src = xb + ((size_t)(r0[s] + idx - H1) * Dc + c) * es;
        memcpy(slot_base + ((size_t)r * Dc + c) * es, src, es);
      }
      if (hb != hist) free(hb);
    }
  }
  free(r0);
  free(sf);
  return ORC_OK;
}

int oracle_conv1d(void* dst, const void* x, const float* w, const float* b, void* conv_state,
                  int S, int T, const int32_t* len, const int32_t* slot, const uint8_t* fresh,
                  int Dc, int K, int M, int act) {
  return conv_impl(dst, x, w, b, conv_state, S, T, len, slot, fresh, Dc, K, M, act, NULL, 0);
}

/* The conv plus its state snapshots every E rows: snaps [count][K-1][Dc] act. */
int oracle_conv1d_snap(void* dst, const void* x, const float* w, const float* b, void* conv_state,
                       int S, int T, const int32_t* len, const int32_t* slot, const uint8_t* fresh,
                       int Dc, int K, int M, int act, void* snaps, int E) {
  return conv_impl(dst, x, w, b, conv_state, S, T, len, slot, fresh, Dc, K, M, act, snaps, E);
}

/* ------------------------------------------------------------------ scan */

/*
 * SSMScan, [gllm#85] "Ops" and "CPU reference": with dt' = softplus(dt +
 * dt_bias) (no clamp: the time-step limit is (0, inf)), each token computes
 *   h = h * exp(-exp(A_log) * dt') + dt' * B (x) x,   y = h . C + D * x,
 * one token at a time, y from the updated h, the state rounded to fp32 after
 * every token.  Head h reads B and C of group h / (H / G).  The state seeds
 * from the sequence's slot (zeros when fresh) and is written back to it.
 * D is one value per head ([InfiniLM#575] "Notes for Reviewers").
 *
 * xbc is the conv output row [x (H*P, head-major) | B (G*N) | C (G*N)].
 * Layouts: xbc [T][Dc] act, Dc = H*P + 2*G*N; dt [T][H] act; a_log, dt_bias,
 * d [H] f32; y [T][H*P] act; ssm_state [M][H][P][N] f32.
 *
 * head_mask (may be NULL) limits the work to the heads whose entry is nonzero;
 * heads are independent, so the selected heads are computed exactly as in a
 * full run, and the others are neither read nor written.
 * decode != 0 applies the decode rule (every run length is 1); the arithmetic
 * is the same function.
 */
static int scan_impl(void* y, const void* xbc, const void* dt, const float* a_log, const float* dt_bias,
                     const float* d, float* ssm_state, int S, int T, const int32_t* len,
                     const int32_t* slot, const uint8_t* fresh, int H, int P, int N, int G, int M,
                     int act, const uint8_t* head_mask, int decode, float* snaps, int E) {
  if (H <= 0 || P <= 0 || N <= 0 || G <= 0 || H % G != 0 || (act != ORC_F32 && act != ORC_BF16))
    return ORC_INVALID_ARGUMENT;
  if (snaps != NULL && E < 1) return ORC_INVALID_ARGUMENT;
  int st = check_batch(S, T, len, slot, M, decode);
  if (st != ORC_OK) return st;
  if (S == 0) return ORC_OK;
  if (fresh == NULL) return ORC_INVALID_ARGUMENT;
  long long* r0 = (long long*)malloc(sizeof(long long) * (size_t)S);
  first_rows(S, len, r0);
  long long* sf = (long long*)malloc(sizeof(long long) * (size_t)S);
  if (snaps != NULL) snap_first(S, len, E, sf);
  const size_t Di = (size_t)H * P;
  const size_t Dc = Di + 2 * (size_t)G * N;
  const int heads_per_group = H / G;

#pragma omp parallel for collapse(2) schedule(dynamic, 1)
  for (int s = 0; s < S; ++s) {
    for (int hh = 0; hh < H; ++hh) {
      if (head_mask && !head_mask[hh]) continue;
      const int g = hh / heads_per_group;
      float* st_slot = ssm_state + ((size_t)slot[s] * H + hh) * (size_t)P * N;
      float* h = (float*)malloc(sizeof(float) * (size_t)P * N);
      if (fresh[s])
        memset(h, 0, sizeof(float) * (size_t)P * N);
      else
        memcpy(h, st_slot, sizeof(float) * (size_t)P * N);
      const double A = exp((double)a_log[hh]);
      for (int t = 0; t < len[s]; ++t) {
        const size_t row = (size_t)(r0[s] + t);
        const double v = load_act(dt, row * H + hh, act) + (double)dt_bias[hh];
        const double dtp = v > 20.0 ? v : log1p(exp(v)); /* softplus */
        const double dA = exp(-A * dtp);
        const size_t boff = row * Dc + Di + (size_t)g * N;
        const size_t coff = row * Dc + Di + (size_t)G * N + (size_t)g * N;
        for (int p = 0; p < P; ++p) {
          const double xv = load_act(xbc, row * Dc + (size_t)hh * P + p, act);
          float* hp = h + (size_t)p * N;
          double acc = 0.0;
          for (int n = 0; n < N; ++n) {
            const double Bn = load_act(xbc, boff + n, act);
            hp[n] = (float)((double)hp[n] * dA + (dtp * xv) * Bn);
          }
          for (int n = 0; n < N; ++n) acc += (double)hp[n] * load_act(xbc, coff + n, act);
          acc += (double)d[hh] * xv;
          store_act(y, row * Di + (size_t)hh * P + p, act, acc);
        }
        /* h is now the state after row t + 1 of the run */
        const int bd = t + 1;
        if (snaps != NULL && bd < len[s] && bd % E == 0)
          memcpy(snaps + ((size_t)(sf[s] + bd / E - 1) * H + hh) * (size_t)P * N, h,
                 sizeof(float) * (size_t)P * N);
      }
      memcpy(st_slot, h, sizeof(float) * (size_t)P * N);
      free(h);
    }
  }
  free(r0);
  free(sf);
  return ORC_OK;
}

int oracle_scan(void* y, const void* xbc, const void* dt, const float* a_log, const float* dt_bias,
                const float* d, float* ssm_state, int S, int T, const int32_t* len,
                const int32_t* slot, const uint8_t* fresh, int H, int P, int N, int G, int M,
                int act, const uint8_t* head_mask, int decode) {
  return scan_impl(y, xbc, dt, a_log, dt_bias, d, ssm_state, S, T, len, slot, fresh, H, P, N, G, M, act,
                   head_mask, decode, NULL, 0);
}

/* The scan plus its state snapshots every E rows: snaps [count][H][P][N] f32. */
int oracle_scan_snap(void* y, const void* xbc, const void* dt, const float* a_log, const float* dt_bias,
                     const float* d, float* ssm_state, int S, int T, const int32_t* len,
                     const int32_t* slot, const uint8_t* fresh, int H, int P, int N, int G, int M,
                     int act, float* snaps, int E) {
  return scan_impl(y, xbc, dt, a_log, dt_bias, d, ssm_state, S, T, len, slot, fresh, H, P, N, G, M, act,
                   NULL, 0, snaps, E);
}

/*
 * Rollback after a verified run (speculative decoding): sequence s accepted the
 * first m = accepted[s] rows of its run.  When 1 <= m < L and m is a boundary
 * (m % E == 0), its slots take the snapshots at m; otherwise (m == L: the slots
 * already hold the state after the run; anything else) they are left as they
 * are.  Either snapshot array may be NULL (that pool is then not touched).
 */
int oracle_commit(float* ssm_state, void* conv_state, const float* ssm_snaps, const void* conv_snaps,
                  int E, const int32_t* accepted, int S, const int32_t* len, const int32_t* slot,
                  int H, int P, int N, int Dc, int K, int act) {
  if (E < 1 || S < 0 || (S > 0 && (accepted == NULL || len == NULL || slot == NULL))) return ORC_INVALID_ARGUMENT;
  long long* sf = (long long*)malloc(sizeof(long long) * (size_t)(S > 0 ? S : 1));
  snap_first(S, len, E, sf);
  const size_t es = act_size(act);
  const size_t spn = (size_t)H * P * N;
  const size_t cst = (size_t)(K - 1) * Dc;
  for (int s = 0; s < S; ++s) {
    const int m = accepted[s];
    if (m < 1 || m >= len[s] || m % E != 0) continue;
    const long long idx = sf[s] + m / E - 1;
    if (ssm_snaps != NULL) memcpy(ssm_state + (size_t)slot[s] * spn, ssm_snaps + (size_t)idx * spn, spn * 4);
    if (conv_snaps != NULL)
      memcpy((unsigned char*)conv_state + (size_t)slot[s] * cst * es,
             (const unsigned char*)conv_snaps + (size_t)idx * cst * es, cst * es);
  }
  free(sf);
  return ORC_OK;
}

/* ------------------------------------------------------------------ norm */

/*
 * GatedRMSNorm, [gllm#85] "Ops": rmsnorm(x * silu(z)) * weight, the gate applied
 * before the norm and the RMS taken per group of d_inner / groups columns:
 *   g_i = x_i * z_i / (1 + exp(-z_i)),  ms = mean over the group of g^2,
 *   out_i = g_i / sqrt(ms + eps) * w_i.
 * Layouts: x, z, dst [rows][Di] act; w [Di] f32.
 */
int oracle_gated_rmsnorm(void* dst, const void* x, const void* z, const float* w, int groups,
                         float eps, int rows, int Di, int act) {
  if (rows < 0 || Di <= 0 || groups <= 0 || Di % groups != 0 || (act != ORC_F32 && act != ORC_BF16))
    return ORC_INVALID_ARGUMENT;
  const int gs = Di / groups;
#pragma omp parallel for schedule(static)
  for (int r = 0; r < rows; ++r) {
    double* g = (double*)malloc(sizeof(double) * (size_t)gs);
    for (int q = 0; q < groups; ++q) {
      double ss = 0.0;
      for (int i = 0; i < gs; ++i) {
        const size_t at = (size_t)r * Di + (size_t)q * gs + i;
        const double zv = load_act(z, at, act);
        g[i] = load_act(x, at, act) * (zv / (1.0 + exp(-zv)));
        ss += g[i] * g[i];
      }
      const double rms = sqrt(ss / (double)gs + (double)eps);
      for (int i = 0; i < gs; ++i) {
        const size_t at = (size_t)r * Di + (size_t)q * gs + i;
        store_act(dst, at, act, g[i] / rms * (double)w[(size_t)q * gs + i]);
      }
    }
    free(g);
  }
  return ORC_OK;
}

/* ------------------------------------------------------------ projections */

/*
 * The projections on either side of the mixer path (a linear layer, one weight
 * row per output feature): dst[m][n] = sum_k x[m][k] * w[n][k], summed in
 * double from the stored values and rounded once to the activation type.
 * Layouts: x [M][K], w [N][K], dst [M][N], all act.
 */
int oracle_linear(void* dst, const void* x, const void* w, int M, int N, int K, int act) {
  if (M < 0 || N < 1 || K < 1 || (act != ORC_F32 && act != ORC_BF16)) return ORC_INVALID_ARGUMENT;
#pragma omp parallel for schedule(static)
  for (int m = 0; m < M; ++m) {
    for (int n = 0; n < N; ++n) {
      double acc = 0.0;
      for (int k = 0; k < K; ++k)
        acc += load_act(x, (size_t)m * K + k, act) * load_act(w, (size_t)n * K + k, act);
      store_act(dst, (size_t)m * N + n, act, acc);
    }
  }
  return ORC_OK;
}

/* --------------------------------------------------------- padded batches */

/*
 * Padded batches: the layer entry of "Granite Mamba2 Inference Optimization"
 * takes hidden states [B][Lmax] with an attention mask and must match across
 * variable-length padded batches.  Reading: mask[b][j] nonzero marks a real
 * row; the real rows of each batch row form one run, at the end of the row for
 * every row (left padding) or at its start for every row (right padding); the
 * run is the sequence (padding rows are not part of it).  A row without real
 * rows, a gap inside a run, or a mix of the two sides is rejected.
 */
int oracle_padded_runs(const uint8_t* mask, int B, int Lmax, int32_t* lens, int32_t* left_padded) {
  if (B < 0 || Lmax < 1 || (B > 0 && (mask == NULL || lens == NULL))) return ORC_INVALID_ARGUMENT;
  int left_ok = 1, right_ok = 1;
  for (int b = 0; b < B; ++b) {
    const uint8_t* m = mask + (size_t)b * Lmax;
    int n = 0, first = -1, last = -1;
    for (int j = 0; j < Lmax; ++j)
      if (m[j]) {
        if (first < 0) first = j;
        last = j;
        ++n;
      }
    if (n == 0 || last - first + 1 != n) return ORC_INVALID_ARGUMENT;
    lens[b] = n;
    if (last != Lmax - 1) left_ok = 0;
    if (first != 0) right_ok = 0;
  }
  if (!left_ok && !right_ok) return ORC_INVALID_ARGUMENT;
  if (left_padded) *left_padded = left_ok && !right_ok ? 1 : 0;
  return ORC_OK;
}

/* First padded position of row b's run. */
static int run_start(int left_padded, int Lmax, int L) { return left_padded ? Lmax - L : 0; }

/* dst[T][row_bytes] <- the real rows of src[B][Lmax][row_bytes], batch row after batch row. */
int oracle_pack_rows(void* dst, const void* src, int B, int Lmax, const int32_t* lens, int left_padded,
                     size_t row_bytes) {
  size_t t = 0;
  for (int b = 0; b < B; ++b) {
    if (lens[b] < 1 || lens[b] > Lmax) return ORC_INVALID_ARGUMENT;
    const int j0 = run_start(left_padded, Lmax, lens[b]);
    for (int i = 0; i < lens[b]; ++i, ++t)
      memcpy((unsigned char*)dst + t * row_bytes,
             (const unsigned char*)src + ((size_t)b * Lmax + j0 + i) * row_bytes, row_bytes);
  }
  return ORC_OK;
}

/* dst[B][Lmax][row_bytes] <- the packed rows at their padded positions, zero bytes on padding. */
int oracle_unpack_rows(void* dst, const void* src, int B, int Lmax, const int32_t* lens, int left_padded,
                       size_t row_bytes) {
  size_t t = 0;
  for (int b = 0; b < B; ++b) {
    if (lens[b] < 1 || lens[b] > Lmax) return ORC_INVALID_ARGUMENT;
    const int j0 = run_start(left_padded, Lmax, lens[b]);
    for (int j = 0; j < Lmax; ++j) {
      unsigned char* d = (unsigned char*)dst + ((size_t)b * Lmax + j) * row_bytes;
      if (j >= j0 && j < j0 + lens[b])
        memcpy(d, (const unsigned char*)src + (t + (size_t)(j - j0)) * row_bytes, row_bytes);
      else
        memset(d, 0, row_bytes);
    }
    t += (size_t)lens[b];
  }
  return ORC_OK;
}

int oracle_max_threads(void) {
#ifdef _OPENMP
  return omp_get_max_threads();
#else
  return 1;
#endif
}

void oracle_set_threads(int n) {
#ifdef _OPENMP
  if (n > 0) omp_set_num_threads(n);
#else
  (void)n;
#endif
}
