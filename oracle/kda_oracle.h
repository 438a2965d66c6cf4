/*
 * kda_oracle.h -- fp64 CPU oracle for the Kimi Delta Attention (KDA) forward
 * pass.  TEST INFRASTRUCTURE ONLY: called from tests/, from the smoke check and
 * from the benchmark's CPU-baseline leg, never from the product path.  It
 * shares no code, header or constant with the HIP library.
 *
 * Definitions followed (cited by page title and section):
 *  - Recurrence, Eq. 1: "Kimi K3: the paper and proofs side by side",
 *    section 2.1.1 (Equation 1): S_t = (I - beta_t k_t k_t^T) Diag(alpha_t)
 *    S_{t-1} + beta_t k_t v_t^T, and the output reads the UPDATED state,
 *    o_t = S_t^T q_t.  The coordinate order (decay rows, read the decayed
 *    state with the key, subtract beta k (x) read, add beta k (x) v) is the
 *    factorised update on that page ("Writing the KDA update as a tensor
 *    function", update / update_get2).
 *  - Gate, Eq. 5: "Kimi K3 reading notes" (jianyuh.github.io), section 2
 *    (Hybrid Attention): g = g_min * Sigmoid(exp(A^h) * z), alpha = exp(g),
 *    g_min = -5.
 *
 * Layouts (row-major, contiguous): q, k, z, g: [B, T, H, dk]; v, o:
 * [B, T, H, dv]; beta: [B, T, H]; A: [H, dk]; states: [B, H, dk, dv] with
 * rows = key channels, columns = value channels.
 */
#ifndef KDA_ORACLE_H
#define KDA_ORACLE_H

#ifdef __cplusplus
extern "C" {
#endif

/* G[b,t,h,c] = sum of g over the tokens of t's chunk up to and including t,
 * chunks of `chunk` tokens starting at t = 0; chunk == 1 gives g itself.
 * Returns 0, or -1 on bad arguments. */
int kda_oracle_gate(const double* z, const double* A, double g_min,
                    long B, long T, long H, long dk, long chunk, double* G);

/* Token-by-token recurrence with per-token log-decay g (alpha = exp(g)).
 * S_in may be NULL (zero state); S_out may be NULL or alias S_in.
 * o = scale * S_t^T q_t.  nthreads <= 0 uses all online cores.
 * Returns 0, or -1 on bad arguments. */
int kda_oracle_recurrence(const double* q, const double* k, const double* v,
                          const double* beta, const double* g,
                          const double* S_in, double* o, double* S_out,
                          long B, long T, long H, long dk, long dv,
                          double scale, int nthreads);

/* Full forward from decay logits: gate (chunk 1) then the recurrence, without
 * materialising g for the whole tensor (each task recomputes its own). */
int kda_oracle_forward_z(const double* q, const double* k, const double* v,
                         const double* beta, const double* z, const double* A,
                         double g_min, const double* S_in, double* o,
                         double* S_out, long B, long T, long H, long dk,
                         long dv, double scale, int nthreads);

#ifdef __cplusplus
}
#endif
#endif
