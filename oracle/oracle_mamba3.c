/*
 * Plain CPU oracle for the Mamba-3 SISO forward over packed variable-length sequences.
 *
 * TEST INFRASTRUCTURE ONLY.  Only the tests, the smoke check and the bench's
 * CPU-baseline leg may load this library.  It shares no code, header, table or
 * helper with the GPU library.
 *
 * Source (page title -> section):
 *   [Mamba-3]  "Mamba-3 SISO Long-Ragged Multi-Chunk Joint States Full VJP",
 *              section "What You Have" (the seven steps the operator takes per
 *              packed sequence; cu_seqlens with everything reset at each
 *              boundary; GQA 1 -> 32, Q/K width 128, V width 64, 32 rotary
 *              angles) and section "Hard Constraints" (the dtypes of the inputs,
 *              of the output and of the four final states).
 *
 * The function below follows those steps in the page's order, one sequence and
 * one head at a time, with the readings the page leaves open (each marked
 * "reading"):
 *   1. the single Q/K head is shared by every value head (GQA 1 -> H);
 *   2. theta = tanh(angles) * pi; the rotary angle of token t is the sum over the
 *      sequence's tokens s <= t of theta_s * dt_s, taken mod 2 pi into [0, 2 pi)
 *      (reading: angles [T, NA] are shared by the heads, dt [T, H] is per head,
 *      so the angle is per (token, head, pair));
 *   3. q + q_bias[h] and k + k_bias[h], then paired rotary embeddings (reading:
 *      pair a < NA is the two adjacent components (2a, 2a + 1), rotated by the
 *      angle of pair a; components from 2 NA on are not rotated);
 *   4. p = sigmoid(trap); dt_next, p_next are the next token's dt and p, zero at
 *      a sequence's last token; shifted_gamma = dt_next (1 - p_next);
 *      scale = dt p + shifted_gamma;
 *   5. the causal decayed QK interaction: y_t = sum_{s <= t} exp(sum_{r = s+1..t}
 *      adt_r) (qh_t . (scale_s kh_s)) v_s (reading: adt is the per-token log of
 *      the decay, added as it is);
 *   6. + d[h] v_t, minus the shifted-QK correction shifted_gamma_t (qh_t . kh_t) v_t,
 *      then the gate: out = y * z * sigmoid(z);
 *   7. per sequence: the final rotary angle (of the last token), the final SSM
 *      state sum_{s} exp(sum_{r = s+1..last} adt_r) scale_s v_s (x) kh_s as
 *      [H][DV][DK] (reading: the outer product the interaction above sums, with
 *      no correction since shifted_gamma is zero at the last token), the final K
 *      state (the last token's biased, rotated key) and the final V state (the
 *      last token's value).
 *
 * Arithmetic in double from the stored inputs; outputs rounded once to their
 * stored type (bf16 round-to-nearest-even through fp32; fp32 round-to-nearest).
 * OpenMP over (sequence, head) pairs, which are independent.
 *
 * Layouts (row-major, last index contiguous): q, k [T][DK] bf16; v, z [T][H][DV]
 * bf16; adt, dt [T][H] f32; trap [T][H] bf16; q_bias, k_bias [H][DK] f32;
 * angles [T][NA] bf16; d [H] f32.  Outputs: out [T][H][DV] bf16; fin_angle
 * [S][H][NA] bf16; fin_ssm [S][H][DV][DK] f32; fin_k [S][H][DK] f32;
 * fin_v [S][H][DV] bf16.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

static double m3_bf16(uint16_t b) {
  uint32_t u = (uint32_t)b << 16;
  float f;
  memcpy(&f, &u, 4);
  return (double)f;
}

static uint16_t m3_to_bf16(double v) {
  float f = (float)v;
  uint32_t u;
  memcpy(&u, &f, 4);
  if ((u & 0x7fffffffu) > 0x7f800000u) return (uint16_t)((u >> 16) | 0x0040u);
  u += 0x7fffu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}

static double m3_sigmoid(double x) { return 1.0 / (1.0 + exp(-x)); }

/* Returns 0, or 1 for malformed sizes / run lengths (nothing written then). */
int oracle_mamba3_forward(uint16_t* out, uint16_t* fin_angle, float* fin_ssm, float* fin_k, uint16_t* fin_v,
                          const uint16_t* q, const uint16_t* k, const uint16_t* v, const float* adt,
                          const float* dt, const uint16_t* trap, const float* q_bias, const float* k_bias,
                          const uint16_t* angles, const float* d, const uint16_t* z, int S, int T,
                          const int32_t* run_lengths, int H, int DK, int DV, int NA) {
  if (S < 0 || T < 0 || H < 1 || DK < 1 || DV < 1 || NA < 0 || 2 * NA > DK) return 1;
  long long sum = 0;
  for (int s = 0; s < S; ++s) {
    if (run_lengths[s] < 1) return 1;
    sum += run_lengths[s];
  }
  if (sum != T) return 1;
  long long* r0 = (long long*)malloc(sizeof(long long) * (S > 0 ? S : 1));
  long long acc = 0;
  for (int s = 0; s < S; ++s) {
    r0[s] = acc;
    acc += run_lengths[s];
  }
  const double two_pi = 2.0 * M_PI;

#pragma omp parallel for collapse(2) schedule(dynamic, 1)
  for (int s = 0; s < S; ++s) {
    for (int h = 0; h < H; ++h) {
      const int L = run_lengths[s];
      const long long b = r0[s];
      double* qh = (double*)malloc(sizeof(double) * (size_t)L * DK);
      double* kh = (double*)malloc(sizeof(double) * (size_t)L * DK);
      double* phi = (double*)malloc(sizeof(double) * (NA > 0 ? NA : 1));
      double* cum = (double*)calloc(NA > 0 ? NA : 1, sizeof(double));
      double* p = (double*)malloc(sizeof(double) * L);
      double* dtv = (double*)malloc(sizeof(double) * L);
      double* ca = (double*)malloc(sizeof(double) * L);
      double* sg = (double*)malloc(sizeof(double) * L);
      double* sc = (double*)malloc(sizeof(double) * L);
      double car = 0.0;
      for (int t = 0; t < L; ++t) {
        const long long r = b + t;
        dtv[t] = (double)dt[r * H + h];
        /* step 2: theta and the running rotary angle, mod 2 pi */
        for (int a = 0; a < NA; ++a) {
          const double theta = tanh(m3_bf16(angles[r * NA + a])) * M_PI;
          cum[a] += theta * dtv[t];
          double ph = fmod(cum[a], two_pi);
          if (ph < 0.0) ph += two_pi;
          phi[a] = ph;
        }
        /* steps 1 and 3: the shared Q/K head, the head's biases, paired rotary */
        for (int n = 0; n < DK; ++n) {
          qh[(size_t)t * DK + n] = m3_bf16(q[r * DK + n]) + (double)q_bias[(size_t)h * DK + n];
          kh[(size_t)t * DK + n] = m3_bf16(k[r * DK + n]) + (double)k_bias[(size_t)h * DK + n];
        }
        for (int a = 0; a < NA; ++a) {
          const double c = cos(phi[a]), sn = sin(phi[a]);
          double* qp = qh + (size_t)t * DK + 2 * a;
          double* kp = kh + (size_t)t * DK + 2 * a;
          const double q0 = qp[0], q1 = qp[1], k0 = kp[0], k1 = kp[1];
          qp[0] = q0 * c - q1 * sn;
          qp[1] = q0 * sn + q1 * c;
          kp[0] = k0 * c - k1 * sn;
          kp[1] = k0 * sn + k1 * c;
        }
        p[t] = m3_sigmoid(m3_bf16(trap[r * H + h]));
        car += (double)adt[r * H + h];
        ca[t] = car;
        if (t == L - 1) {
          for (int a = 0; a < NA; ++a) fin_angle[((size_t)s * H + h) * NA + a] = m3_to_bf16(phi[a]);
        }
      }
      /* step 4: the shifted next-token values, shifted_gamma and scale */
      for (int t = 0; t < L; ++t) {
        const double dt_next = t + 1 < L ? dtv[t + 1] : 0.0;
        const double p_next = t + 1 < L ? p[t + 1] : 0.0;
        sg[t] = dt_next * (1.0 - p_next);
        sc[t] = dtv[t] * p[t] + sg[t];
      }
      /* steps 5 and 6 */
      double* y = (double*)malloc(sizeof(double) * DV);
      for (int t = 0; t < L; ++t) {
        const long long r = b + t;
        for (int e = 0; e < DV; ++e) y[e] = 0.0;
        for (int j = 0; j <= t; ++j) {
          double g = 0.0;
          for (int n = 0; n < DK; ++n) g += qh[(size_t)t * DK + n] * kh[(size_t)j * DK + n];
          const double wgt = exp(ca[t] - ca[j]) * g * sc[j];
          const uint16_t* vj = v + ((b + j) * H + h) * DV;
          for (int e = 0; e < DV; ++e) y[e] += wgt * m3_bf16(vj[e]);
        }
        double gtt = 0.0;
        for (int n = 0; n < DK; ++n) gtt += qh[(size_t)t * DK + n] * kh[(size_t)t * DK + n];
        const uint16_t* vt = v + (r * H + h) * DV;
        const uint16_t* zt = z + (r * H + h) * DV;
        for (int e = 0; e < DV; ++e) {
          const double ve = m3_bf16(vt[e]);
          const double ye = y[e] + (double)d[h] * ve - sg[t] * gtt * ve;
          const double ze = m3_bf16(zt[e]);
          out[(r * H + h) * DV + e] = m3_to_bf16(ye * ze * m3_sigmoid(ze));
        }
      }
      /* step 7: the final states of the sequence */
      {
        const int tl = L - 1;
        float* st = fin_ssm + ((size_t)s * H + h) * (size_t)DV * DK;
        for (int e = 0; e < DV; ++e)
          for (int n = 0; n < DK; ++n) {
            double acc2 = 0.0;
            for (int j = 0; j < L; ++j)
              acc2 += exp(ca[tl] - ca[j]) * sc[j] * m3_bf16(v[((b + j) * H + h) * DV + e]) * kh[(size_t)j * DK + n];
            st[(size_t)e * DK + n] = (float)acc2;
          }
        for (int n = 0; n < DK; ++n) fin_k[((size_t)s * H + h) * DK + n] = (float)kh[(size_t)tl * DK + n];
        for (int e = 0; e < DV; ++e) fin_v[((size_t)s * H + h) * DV + e] = v[((b + tl) * H + h) * DV + e];
      }
      free(y);
      free(qh);
      free(kh);
      free(phi);
      free(cum);
      free(p);
      free(dtv);
      free(ca);
      free(sg);
      free(sc);
    }
  }
  free(r0);
  return 0;
}
