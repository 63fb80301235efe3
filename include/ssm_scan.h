/*
 * ssm_scan.h -- C ABI of libssmscan, a selective state-space scan for AMD
 * Instinct MI355X (gfx950).
 *
 * What the library computes
 * -------------------------
 * The linear state-space recurrence of "Jamba — SSM-Transformer Híbrido"
 * (ai-engineering.academy), section "Um SSM em uma página":
 *     h_t = Abar_t h_{t-1} + Bbar_t x_t,      y_t = C_t h_t,
 * made selective (A, B, C and the step dt depend on the data), with the
 * discretisation, skip term and gate of the MambaBlock on
 * "【大模型】- Jamba 混合 SSM-Transformer", section 4.1 "Mamba 层":
 *     Abar = exp(dt * A)  (A diagonal: one value per channel d and state n)
 *     Bbar = dt * B       (B and C are shared by all channels of a (batch, step))
 *     y    = (sum_n C[n] h[n] + D[d] x) * silu(z),    silu(z) = z / (1 + exp(-z)).
 * The state h is fp32 and its size does not depend on the sequence length
 * (same page, section "O orçamento de memória"). The complex variants (_c64)
 * take A = -a + i*theta per (d, n), so Abar is a decay times a data-dependent
 * rotation (Mamba-3 item on complex-valued state updates, same pt page), and
 * output y = Re(sum_n C[n] h[n]) + D x, then the optional gate.
 * dt is taken after softplus (the MambaBlock applies softplus before its scan), so
 * dt >= 0 is part of the input contract; with dt >= 0 and Re A < 0 the decay of
 * the state only grows with distance in time, which the chunked prefill uses (see
 * ssm_scan_fwd). Negative dt is outside the contract.
 *
 * Conventions (all entry points)
 * ------------------------------
 *  - Every array pointer is a DEVICE pointer owned by the caller; the library
 *    never allocates, frees or retains caller memory. Arrays are contiguous,
 *    row-major, channel index fastest.
 *  - io selects the element type of x, dt, z, B, C and y: SSM_F32 (float) or
 *    SSM_BF16 (bfloat16, stored as 16 bits; y is rounded to nearest even).
 *    A, D and every state (h, h0, h_final) are always float32.
 *  - Alignment: A, h, h0 and h_final 16 bytes; the workspace 256 bytes; B and C
 *    4 bytes for prefill (their rows are read as 32-bit words: with bf16 and an
 *    odd number of elements the last word is read whole), and for real-state
 *    decode min(d_state, 4) elements (read as vectors), element-aligned for
 *    complex decode; D 4 bytes; x, dt, z, y element-aligned.
 *  - d_state must be 1, 2, 4, 8 or 16.
 *  - Work is enqueued on hip_stream (a hipStream_t; NULL = the null stream) and
 *    runs asynchronously; the call returns once it is enqueued.
 *  - Errors: argument errors return a status before anything is enqueued and
 *    leave every output untouched. A failed launch returns SSM_ERR_HIP. NaN or
 *    Inf in the data are not errors; they stay inside their channel.
 *    ssm_last_error() gives a per-thread detail string for the last failure.
 *  - The library keeps no state besides a per-thread error string. Calls that
 *    share no output or workspace memory may run concurrently.
 */
#ifndef SSM_SCAN_H
#define SSM_SCAN_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    SSM_OK = 0,
    SSM_ERR_NULL = 1,         /* a required pointer is NULL */
    SSM_ERR_SHAPE = 2,        /* a size is negative, zero where it must not be, or too large */
    SSM_ERR_DTYPE = 3,        /* io is not SSM_F32 or SSM_BF16 */
    SSM_ERR_ALIGN = 4,        /* a pointer breaks the alignment rules above */
    SSM_ERR_UNSUPPORTED = 5,  /* d_state not in {1, 2, 4, 8, 16}, chunk_len or conv_k invalid,
                                 or a forbidden overlap (fused prefill) */
    SSM_ERR_WORKSPACE = 6,    /* workspace missing or smaller than the query says */
    SSM_ERR_HIP = 7           /* the HIP runtime reported an error at launch */
} ssm_status;

typedef enum { SSM_F32 = 0, SSM_BF16 = 1 } ssm_dtype;

/* ------------------------------------------------------------------ prefill
 * ssm_scan_fwd: the whole recurrence over L steps for every (batch, channel).
 *   x, dt, z, y : [batch, L, d_inner] of io      B, C : [batch, L, d_state] of io
 *   A           : [d_inner, d_state] float32     D    : [d_inner] float32
 *   h0          : [batch, d_inner, d_state] float32, NULL = zero initial state
 *   h_final     : [batch, d_inner, d_state] float32, NULL = not wanted
 *   z           : NULL = no gate (y = C.h + D x)
 * The sequence is split into chunks that run in parallel; each chunk's end state
 * from zero and its total decay are combined across chunks by an associative
 * scan, and each chunk is then re-walked from its true incoming state. This is an
 * exact re-association of the recurrence; results differ from a sequential fp32
 * loop only by rounding and by one bounded truncation: a chunk's end state is
 * accumulated only over its last steps back to the point where the decay
 * exp(Re A * sum of dt) of every state of 64 neighbouring channels is below 2^-H,
 * H = 28 + the bit length of chunk_len (41 for chunks of 4096 to 8191 steps). What is
 * dropped changes a carried state by at most 2^-H * (chunk_len * max|dt x B| +
 * |incoming state|), which is at most 2^-28 of the input scale for every chunk length,
 * below fp32 resolution. NaN or Inf older than that window do not propagate past the
 * chunk boundary. workspace must hold ssm_scan_fwd_workspace(...) bytes
 * (0 is possible, then workspace may be NULL). It is scratch: contents on entry
 * are ignored and on return are unspecified. L == 0 writes h_final = h0 (or
 * zeros) and nothing else. */
size_t ssm_scan_fwd_workspace(int64_t batch, int64_t L, int64_t d_inner, int32_t d_state);

ssm_status ssm_scan_fwd(const void *x, const void *dt, const float *A, const void *B,
                        const void *C, const float *D, const void *z, const float *h0,
                        void *y, float *h_final,
                        int64_t batch, int64_t L, int64_t d_inner, int32_t d_state,
                        ssm_dtype io, void *workspace, size_t workspace_bytes,
                        void *hip_stream);

/* Same, with an explicit chunk length (steps per chunk; 0 = the library's own
 * choice, which is what ssm_scan_fwd uses). chunk_len >= L gives one chunk and
 * needs no workspace. The chunk length is capped so that one chunk spans less than
 * 2 GiB of a [L, d_inner] stream at 4 bytes per element. Results for different
 * chunk lengths agree within rounding. */
size_t ssm_scan_fwd_workspace_ex(int64_t batch, int64_t L, int64_t d_inner, int32_t d_state,
                                 int64_t chunk_len);
ssm_status ssm_scan_fwd_ex(const void *x, const void *dt, const float *A, const void *B,
                           const void *C, const float *D, const void *z, const float *h0,
                           void *y, float *h_final,
                           int64_t batch, int64_t L, int64_t d_inner, int32_t d_state,
                           ssm_dtype io, int64_t chunk_len, void *workspace,
                           size_t workspace_bytes, void *hip_stream);

/* ssm_scan_fwd_noalloc: ssm_scan_fwd_ex for callers that cannot allocate device memory
 * (code under HIP graph capture, tight serving loops, harnesses that forbid hipMalloc).
 * It takes no workspace and calls no allocating routine: the chunk summaries live in a
 * scratch array of SSM_NOALLOC_SCRATCH_BYTES (64 MiB) that the library's code object
 * holds on every GPU it runs on, from the first use on that GPU until the process ends
 * (its device address is looked up once per device). Same arguments, kernels, results
 * and errors as ssm_scan_fwd_ex on the current device (hip_stream must belong to it),
 * plus SSM_ERR_WORKSPACE, before anything is enqueued, when the plan needs more scratch
 * than that: ssm_scan_fwd_workspace_ex(batch, L, d_inner, d_state, chunk_len) >
 * SSM_NOALLOC_SCRATCH_BYTES. The library's own plan (chunk_len = 0) needs less than
 * 2 * (5 waves per SIMD * SIMDs) * 64 * d_state * 4 bytes: 42 MB at d_state 16 on the
 * 1024 SIMDs of MI355X, which fits. Calls on one
 * GPU share its scratch, and nothing in it needs to start cleared (each call writes
 * every summary before reading it); calls that overlap in time on one GPU (on
 * different streams, or from different threads) race on it and must be ordered by the
 * caller. */
#define SSM_NOALLOC_SCRATCH_BYTES (64u << 20)
ssm_status ssm_scan_fwd_noalloc(const void *x, const void *dt, const float *A, const void *B,
                                const void *C, const float *D, const void *z, const float *h0,
                                void *y, float *h_final,
                                int64_t batch, int64_t L, int64_t d_inner, int32_t d_state,
                                ssm_dtype io, int64_t chunk_len, void *hip_stream);

/* The chunk length each prefill entry point picks for this shape with chunk_len = 0
 * (host functions; 0 for an invalid shape). The plan is made for the current device: its
 * compute-unit count is queried once per device (hipDeviceGetAttribute) and cached for
 * the process; a positive integer in the environment variable SSMSCAN_CU_COUNT at that
 * first query replaces it (to plan for another part or partition), and with no device
 * to query the plan assumes MI355X's 256 compute units (1024 SIMDs), uncached. The
 * library cuts the sequence into
 * enough chunks to keep as many waves per SIMD resident as the entry point's rescan
 * kernel is compiled for: 5 for ssm_scan_fwd / _ex / _trap (with or without lam),
 * ssm_scan_fwd_c64 (whose channels take 4 lanes each) and ssm_scan_fwd_mimo up to rank
 * 4; 4 for ssm_scan_fwd_fused and rank 8 (and the backward). ssm_scan_fwd_trap uses the
 * plan of ssm_scan_fwd_chunk_len.
 * A plan with fewer chunks needs no more workspace, so ssm_scan_fwd_workspace_ex(...,
 * 0) also suffices for ssm_scan_fwd_fused. */
int64_t ssm_scan_fwd_chunk_len(int64_t batch, int64_t L, int64_t d_inner, int32_t d_state);
int64_t ssm_scan_fwd_fused_chunk_len(int64_t batch, int64_t L, int64_t d_inner, int32_t d_state);
int64_t ssm_scan_fwd_c64_chunk_len(int64_t batch, int64_t L, int64_t d_inner, int32_t d_state);
int64_t ssm_scan_fwd_mimo_chunk_len(int64_t batch, int64_t L, int64_t d_inner, int32_t d_state,
                                    int32_t rank);

/* ------------------------------------------------------------------ decode
 * ssm_step: one token for every (layer, sequence, channel); h -> h' in place.
 * Each layer's state needs only the previous state and the new token
 * ("Um SSM em uma página": constant memory, O(1) per token).
 *   h              : [n_layers, n_seq, d_inner, d_state] float32 (read and written)
 *   x_t, dt_t, z_t : [n_layers, n_seq, d_inner] of io;  y_t: same shape, written
 *   B_t, C_t       : [n_layers, n_seq, d_state] of io
 *   A              : [n_layers, d_inner, d_state] float32;  D: [n_layers, d_inner]
 *   z_t            : NULL = no gate
 * n_layers and n_seq are at most 65535 each, d_inner at most 2^28.
 * Per channel the fp32 operations are, in this order (fma = fused multiply-add,
 * e2 = the hardware base-2 exponential, G = d_state >= 8 ? d_state / 4 : 1 groups
 * of K = d_state / G states):
 *   xf, dtf, zf widened; u = dtf * xf
 *   for each group g: p_g = 0; for k in group: a = A[n] * log2(e);
 *       h[n] = fma(e2(dtf * a), h[n], u * Bf[n]); p_g = fma(Cf[n], h[n], p_g)
 *   acc = pairwise sum of the p_g ((p0 + p1) + (p2 + p3) for G = 4)
 *   y = fma(D, xf, acc); gated: y = y * (zf * rcp(1 + e2(-zf * log2(e))))
 * ssm_step_replay performs exactly this sequence with one thread per channel and
 * plain loops; it exists so that the decode kernel can be checked bit for bit. */
ssm_status ssm_step(float *h, const void *x_t, const void *dt_t, const float *A,
                    const void *B_t, const void *C_t, const float *D, const void *z_t,
                    void *y_t, int64_t n_layers, int64_t n_seq, int64_t d_inner,
                    int32_t d_state, ssm_dtype io, void *hip_stream);

ssm_status ssm_step_replay(float *h, const void *x_t, const void *dt_t, const float *A,
                           const void *B_t, const void *C_t, const float *D, const void *z_t,
                           void *y_t, int64_t n_layers, int64_t n_seq, int64_t d_inner,
                           int32_t d_state, ssm_dtype io, void *hip_stream);

/* ------------------------------------------------------------------ complex state
 * As above with a complex diagonal state. Complex values are (re, im) float
 * pairs, the pair index fastest:
 *   A        : [d_inner, d_state, 2] float32, A = (-a, theta): Abar = exp(dt * A)
 *   B, C     : [batch, L, d_state, 2] of io (decode: [n_layers, n_seq, d_state, 2])
 *   h0, h_final, h : [..., d_state, 2] float32
 *   y = Re(sum_n C[n] h[n]) + D x (C not conjugated), then the optional gate.
 * Decode groups: G = d_state >= 2 ? d_state / 2 : 1 lanes of K = d_state / G
 * complex states, partial sums combined pairwise as in ssm_step. */
size_t ssm_scan_fwd_c64_workspace(int64_t batch, int64_t L, int64_t d_inner, int32_t d_state,
                                  int64_t chunk_len);
ssm_status ssm_scan_fwd_c64(const void *x, const void *dt, const float *A, const void *B,
                            const void *C, const float *D, const void *z, const float *h0,
                            void *y, float *h_final,
                            int64_t batch, int64_t L, int64_t d_inner, int32_t d_state,
                            ssm_dtype io, int64_t chunk_len, void *workspace,
                            size_t workspace_bytes, void *hip_stream);
ssm_status ssm_step_c64(float *h, const void *x_t, const void *dt_t, const float *A,
                        const void *B_t, const void *C_t, const float *D, const void *z_t,
                        void *y_t, int64_t n_layers, int64_t n_seq, int64_t d_inner,
                        int32_t d_state, ssm_dtype io, void *hip_stream);
ssm_status ssm_step_c64_replay(float *h, const void *x_t, const void *dt_t, const float *A,
                               const void *B_t, const void *C_t, const float *D,
                               const void *z_t, void *y_t, int64_t n_layers, int64_t n_seq,
                               int64_t d_inner, int32_t d_state, ssm_dtype io,
                               void *hip_stream);

/* ------------------------------------------------------------------ fused input stage
 * Between its input projection and its scan, the MambaBlock ("【大模型】- Jamba 混合
 * SSM-Transformer", section 4.1 "Mamba 层") computes
 *     u  = silu(conv(x_in)),   conv = a causal depthwise convolution over time:
 *          conv(x)_t[d] = conv_b[d] + sum_{k<K} conv_w[d][k] * x_{t-(K-1)+k}[d]
 *          (K = conv_k taps; K-1 zeros of padding in front, output cut back to L steps;
 *          inputs before step 0 come from the carried conv state)
 *     dt = softplus(dt_raw + dt_bias),   softplus(v) = log(1 + e^v)
 *          (dt_raw is the dt projection's output without its bias)
 * and scans with u in place of x (the skip term uses u as well). These entry points
 * apply both while loading x_in and dt_raw, so neither u nor dt is ever written to
 * memory. Real state only; the recurrence, gate and outputs are those of
 * ssm_scan_fwd / ssm_step, and dt >= 0 holds by construction.
 *   conv_k        0 = no convolution (x_in is used as is and the conv pointers are
 *                 ignored), else 1..4 (the page's d_conv is 4). Other values:
 *                 SSM_ERR_UNSUPPORTED.
 *   conv_w        [d_inner, conv_k] float32 (decode: [n_layers, d_inner, conv_k]);
 *                 required when conv_k > 0.
 *   conv_b        [d_inner] float32 (decode: [n_layers, d_inner]); NULL = no bias.
 *   dt_bias       [d_inner] float32 (decode: [n_layers, d_inner]); NULL = 0.
 *   conv state    the last conv_k-1 inputs x_in, oldest first, in the io type:
 *                 prefill [batch, conv_k-1, d_inner], decode [n_layers, n_seq,
 *                 conv_k-1, d_inner]. Alignment: one element; conv_w, conv_b, dt_bias
 *                 4 bytes.
 * Inside the kernels: dt as e = e2(-|v| log2 e), w = 1 + e, l = (w == 1) ? e :
 * (log2(w) ln 2) (e rcp(w - 1)) (Goldberg's log1p correction), dt = max(v, 0) + l
 * for v = dt_raw + dt_bias; u as acc = conv_b, acc = fma(conv_w[k], input, acc) for
 * k ascending, u = acc rcp(1 + e2(-acc log2 e)).
 *
 * ssm_scan_fwd_fused: prefill. conv_state0 NULL = zeros before step 0 (the page's
 * padding). conv_state_out NULL = not wanted; else it receives the last conv_k-1
 * inputs (from conv_state0 where L < conv_k-1). workspace: ssm_scan_fwd_workspace_ex
 * bytes for the same shape and chunk_len (enough for its own plan when chunk_len is 0:
 * see ssm_scan_fwd_fused_chunk_len). With conv_k > 1, y must not overlap x_in
 * (a chunk reads the previous chunk's last inputs), and conv_state_out must not
 * overlap x_in or conv_state0: SSM_ERR_UNSUPPORTED otherwise. L == 0 writes
 * h_final = h0 and conv_state_out = conv_state0 (or zeros). */
ssm_status ssm_scan_fwd_fused(const void *x_in, const void *dt_raw, const float *A, const void *B,
                              const void *C, const float *D, const void *z, const float *h0,
                              const float *conv_w, const float *conv_b, int32_t conv_k,
                              const void *conv_state0, void *conv_state_out,
                              const float *dt_bias, void *y, float *h_final,
                              int64_t batch, int64_t L, int64_t d_inner, int32_t d_state,
                              ssm_dtype io, int64_t chunk_len, void *workspace,
                              size_t workspace_bytes, void *hip_stream);

/* ssm_step_fused: one decode token; h and conv_state (required when conv_k > 1) are
 * updated in place. x_t is the convolution's new input and dt_t the raw dt.
 * ssm_step_fused_replay: the same in the written-down order, one thread per channel
 * (bit-for-bit reference for ssm_step_fused). */
ssm_status ssm_step_fused(float *h, void *conv_state, const void *x_t, const void *dt_t,
                          const float *A, const void *B_t, const void *C_t, const float *D,
                          const void *z_t, const float *conv_w, const float *conv_b,
                          int32_t conv_k, const float *dt_bias, void *y_t, int64_t n_layers,
                          int64_t n_seq, int64_t d_inner, int32_t d_state, ssm_dtype io,
                          void *hip_stream);
ssm_status ssm_step_fused_replay(float *h, void *conv_state, const void *x_t, const void *dt_t,
                                 const float *A, const void *B_t, const void *C_t, const float *D,
                                 const void *z_t, const float *conv_w, const float *conv_b,
                                 int32_t conv_k, const float *dt_bias, void *y_t,
                                 int64_t n_layers, int64_t n_seq, int64_t d_inner,
                                 int32_t d_state, ssm_dtype io, void *hip_stream);

/* ------------------------------------------------------------------ backward
 * ssm_scan_bwd: gradients of the real-state prefill, for training. Given the
 * forward's inputs and the upstream gradients dy = dLoss/dy [batch, L, d_inner] (io)
 * and dh_final = dLoss/dh_final [batch, d_inner, d_state] float32 (NULL = 0), it
 * writes the gradients of Loss = sum(dy * y) + sum(dh_final * h_final):
 *   dx, ddt, dz : [batch, L, d_inner] of io (dz only when z is given; NULL = not wanted)
 *   dA          : [d_inner, d_state] float32 (summed over batch and steps)
 *   dB, dC      : [batch, L, d_state] float32 (summed over channels)
 *   dD          : [d_inner] float32;   dh0: [batch, d_inner, d_state] float32 (NULL = not wanted)
 * It is the chain rule through the recurrence of ssm_scan_fwd ("Jamba — SSM-Transformer
 * Híbrido", section "Um SSM em uma página"; gate and skip of the MambaBlock,
 * "【大模型】- Jamba 混合 SSM-Transformer", section 4.1): the adjoint
 * lam_t = dLoss/dh_t = do_t C_t + exp(dt_{t+1} A) lam_{t+1} with do_t = dy_t silu(z_t)
 * runs backwards, and dx_t = do_t D + dt_t lam_t.B_t, ddt_t = lam_t.(x_t B_t + A a_t h_{t-1}),
 * dz_t = dy_t o_t silu'(z_t), dA += dt_t lam_t a_t h_{t-1}, dB_t += lam_t dt_t x_t,
 * dC_t += do_t h_t, dD += do_t x_t, dh0 = a_0 lam_0 (o_t = C_t.h_t + D x_t before the
 * gate, a_t = exp(dt_t A)).
 * The states are recomputed: chunked as in the forward (the same decay-horizon
 * truncation, applied to the state and, mirrored, to the adjoint), with the state
 * stored every 8 steps in the workspace and each 4-step piece recomputed in
 * registers. The workspace (ssm_scan_bwd_workspace bytes, 256-byte aligned) holds
 * those states (8 bytes per element at N = 16, fp32) and per-chunk and per-wave
 * partial sums; dA, dB, dC and dD are reduced from them in a fixed order, so results
 * are deterministic. chunk_len: as in ssm_scan_fwd_ex (rounded down to a multiple of
 * 4 when there are several chunks). L == 0: dA = dD = 0, dh0 = dh_final (or 0).
 * SSM_ERR_UNSUPPORTED when batch * d_inner * d_state * 4 bytes (one state array) is
 * 2 GiB or more. Alignment: A, h0, dh_final, dh0 16 bytes; B, C, D, dA, dB, dC, dD
 * 4 bytes; streams one element; workspace 256 bytes. */
size_t ssm_scan_bwd_workspace(int64_t batch, int64_t L, int64_t d_inner, int32_t d_state,
                              int64_t chunk_len);
ssm_status ssm_scan_bwd(const void *x, const void *dt, const float *A, const void *B,
                        const void *C, const float *D, const void *z, const float *h0,
                        const void *dy, const float *dh_final, void *dx, void *ddt, void *dz,
                        float *dA, float *dB, float *dC, float *dD, float *dh0,
                        int64_t batch, int64_t L, int64_t d_inner, int32_t d_state,
                        ssm_dtype io, int64_t chunk_len, void *workspace,
                        size_t workspace_bytes, void *hip_stream);

/* Training with stored states: ssm_scan_fwd_save is ssm_scan_fwd_ex that also writes the
 * state entering every 8th step to `states` (caller-owned device memory of
 * ssm_scan_fwd_save_states_bytes: ceil(L / 8) rows of batch * d_inner * d_state fp32, row
 * r the state entering step 8 r, row 0 h0 or zeros; within a row, for d_state a multiple
 * of 4, [batch][d_state / 4][d_inner][4], else [batch][d_inner][d_state]). y and h_final
 * equal ssm_scan_fwd_ex's bit for bit for the same chunk length; with several chunks the
 * chunk length is rounded down to a multiple of 8 (at least 8), and the workspace is
 * ssm_scan_fwd_save_workspace bytes. ssm_scan_bwd_saved is ssm_scan_bwd given those
 * states instead of h0: it reads them where ssm_scan_bwd recomputes them by a forward
 * walk of every chunk (the forward's chunk summaries, the carry over them and that walk
 * are skipped), and its workspace (ssm_scan_bwd_saved_workspace) holds no states; its
 * chunk length is rounded the same way. The states must come from ssm_scan_fwd_save on
 * the same x, dt, A, B and h0 and be unchanged since. The stored states (8 bytes per
 * element at d_state = 16) cost the forward their writes; the backward saves its walk:
 * at batch 1, L = 262144, d_inner = 8192 they are 17 GB. SSM_ERR_UNSUPPORTED when a state
 * row (batch * d_inner * d_state * 4 bytes) is 2 GiB or more; SSM_ERR_NULL without
 * states (L > 0); states 16-byte aligned, other arguments as in ssm_scan_fwd_ex and
 * ssm_scan_bwd. Floating point: the backward reads the states the forward computed, so
 * its gradients agree with ssm_scan_bwd's to rounding, not bit for bit. */
size_t ssm_scan_fwd_save_states_bytes(int64_t batch, int64_t L, int64_t d_inner, int32_t d_state);
size_t ssm_scan_fwd_save_workspace(int64_t batch, int64_t L, int64_t d_inner, int32_t d_state,
                                   int64_t chunk_len);
ssm_status ssm_scan_fwd_save(const void *x, const void *dt, const float *A, const void *B,
                             const void *C, const float *D, const void *z, const float *h0,
                             void *y, float *h_final, float *states, int64_t batch, int64_t L,
                             int64_t d_inner, int32_t d_state, ssm_dtype io, int64_t chunk_len,
                             void *workspace, size_t workspace_bytes, void *hip_stream);
size_t ssm_scan_bwd_saved_workspace(int64_t batch, int64_t L, int64_t d_inner, int32_t d_state,
                                    int64_t chunk_len);
ssm_status ssm_scan_bwd_saved(const void *x, const void *dt, const float *A, const void *B,
                              const void *C, const float *D, const void *z, const float *states,
                              const void *dy, const float *dh_final, void *dx, void *ddt, void *dz,
                              float *dA, float *dB, float *dC, float *dD, float *dh0, int64_t batch,
                              int64_t L, int64_t d_inner, int32_t d_state, ssm_dtype io,
                              int64_t chunk_len, void *workspace, size_t workspace_bytes,
                              void *hip_stream);

/* ssm_scan_bwd_fused: gradients of ssm_scan_fwd_fused's prefill, for training: the
 * backward above on u = silu(conv(x_in)) and dt = softplus(dt_raw + dt_bias), then the
 * chain rule back through the input stage ("【大模型】- Jamba 混合 SSM-Transformer",
 * section 4.1 "Mamba 层": the causal depthwise convolution and silu on x, softplus on
 * the dt projection's output). With xe the conv_k-1 carried inputs followed by x_in,
 * a_t = conv_b + sum_k conv_w[k] xe_{t-(K-1)+k} and da_t = du_t silu'(a_t):
 *   dx_in [batch, L, d_inner] (io):  dx_in_s = sum_k conv_w[k] da_{s+(K-1)-k}
 *   ddt_raw [batch, L, d_inner] (io): ddt_t / (1 + exp(-(dt_raw_t + dt_bias)))
 *   dconv_w [d_inner, conv_k], dconv_b, ddt_bias [d_inner] float32: sums over batch and
 *     steps of da_t xe_{t-(K-1)+k}, da_t and ddt_raw_t (dconv_b, ddt_bias NULL = not
 *     wanted; dconv_w required when conv_k > 0)
 *   dconv_state0 [batch, conv_k-1, d_inner] (io, NULL = not wanted): the gradient of
 *     the carried inputs before step 0 (also when conv_state0 is NULL, i.e. zeros)
 *   dz, dA, dB, dC, dD, dh0: as ssm_scan_bwd.
 * conv_k = 0: no convolution and no silu (u = x_in; dx_in = du). Arguments, layouts and
 * alignment of the forward inputs are those of ssm_scan_fwd_fused (conv_state_out has
 * no counterpart), the rest those of ssm_scan_bwd; dconv_w, dconv_b, ddt_bias 4 bytes,
 * dconv_state0 one element. dx_in must not overlap x_in (SSM_ERR_UNSUPPORTED).
 * u and dt are written in io to the workspace (ssm_scan_bwd_fused_workspace bytes,
 * 256-byte aligned: the scan backward's, then u, dt, du, ddt of batch * L * d_inner
 * elements each, then per-chunk partial sums), so with bf16 io the scan backward sees
 * them rounded to bf16 as ssm_scan_bwd would see bf16 inputs; the input stage's own
 * arithmetic is fp32. The sums are reduced in a fixed order: results are
 * deterministic. L == 0: dconv_w, dconv_b, ddt_bias and dconv_state0 are 0. */
size_t ssm_scan_bwd_fused_workspace(int64_t batch, int64_t L, int64_t d_inner, int32_t d_state,
                                    int32_t conv_k, ssm_dtype io, int64_t chunk_len);
ssm_status ssm_scan_bwd_fused(const void *x_in, const void *dt_raw, const float *A, const void *B,
                              const void *C, const float *D, const void *z, const float *h0,
                              const float *conv_w, const float *conv_b, int32_t conv_k,
                              const void *conv_state0, const float *dt_bias, const void *dy,
                              const float *dh_final, void *dx_in, void *ddt_raw, void *dz,
                              float *dA, float *dB, float *dC, float *dD, float *dh0,
                              float *dconv_w, float *dconv_b, float *ddt_bias, void *dconv_state0,
                              int64_t batch, int64_t L, int64_t d_inner, int32_t d_state,
                              ssm_dtype io, int64_t chunk_len, void *workspace,
                              size_t workspace_bytes, void *hip_stream);

/* Training the fused prefill with stored states: ssm_scan_fwd_fused_save is
 * ssm_scan_fwd_fused that also writes the scan's state entering every 8th step to
 * `states`, in ssm_scan_fwd_save's layout and size (ssm_scan_fwd_save_states_bytes; its
 * chunks rounded as ssm_scan_fwd_save rounds them, and ssm_scan_fwd_save_workspace bytes
 * of workspace suffice), and the scan's inputs as the input stage makes them, u =
 * silu(conv(x_in)) to u_out and dt = softplus(dt_raw + dt_bias) to dt_out ([batch][L]
 * [d_inner] of io each, rounded to io as ssm_scan_bwd_fused rounds them; neither may
 * overlap x_in, dt_raw, y or the other: SSM_ERR_UNSUPPORTED). ssm_scan_bwd_fused_saved
 * is ssm_scan_bwd_fused given those states (instead of h0), u and dt: the scan's backward
 * reads the states as ssm_scan_bwd_saved does and runs on the given u and dt, so the
 * input stage is not evaluated again before it; ssm_scan_bwd_fused_saved_workspace bytes
 * of workspace (no u and dt of its own). The gradients agree with ssm_scan_bwd_fused's
 * to rounding (the stored states come from the forward's unrounded u and dt, the
 * recomputed ones from the rounded); u and dt must not overlap dx_in, ddt_raw or dz
 * (SSM_ERR_UNSUPPORTED). Errors as in the fused and stored-state entry points above;
 * states, u_out and dt_out (u and dt) are required when batch * L > 0. */
ssm_status ssm_scan_fwd_fused_save(const void *x_in, const void *dt_raw, const float *A, const void *B,
                                   const void *C, const float *D, const void *z, const float *h0,
                                   const float *conv_w, const float *conv_b, int32_t conv_k,
                                   const void *conv_state0, void *conv_state_out,
                                   const float *dt_bias, void *y, float *h_final, float *states,
                                   void *u_out, void *dt_out, int64_t batch, int64_t L,
                                   int64_t d_inner, int32_t d_state, ssm_dtype io,
                                   int64_t chunk_len, void *workspace, size_t workspace_bytes,
                                   void *hip_stream);
size_t ssm_scan_bwd_fused_saved_workspace(int64_t batch, int64_t L, int64_t d_inner,
                                          int32_t d_state, int32_t conv_k, ssm_dtype io,
                                          int64_t chunk_len);
ssm_status ssm_scan_bwd_fused_saved(const void *x_in, const void *dt_raw, const float *A,
                                    const void *B, const void *C, const float *D, const void *z,
                                    const float *states, const void *u, const void *dt,
                                    const float *conv_w, const float *conv_b,
                                    int32_t conv_k, const void *conv_state0, const float *dt_bias,
                                    const void *dy, const float *dh_final, void *dx_in,
                                    void *ddt_raw, void *dz, float *dA, float *dB, float *dC,
                                    float *dD, float *dh0, float *dconv_w, float *dconv_b,
                                    float *ddt_bias, void *dconv_state0, int64_t batch, int64_t L,
                                    int64_t d_inner, int32_t d_state, ssm_dtype io,
                                    int64_t chunk_len, void *workspace, size_t workspace_bytes,
                                    void *hip_stream);

/* ------------------------------------------------------------------ exponential-trapezoidal
 * ssm_scan_fwd_trap: the prefill of ssm_scan_fwd_ex with the exponential-trapezoidal
 * discretisation that Mamba-3 puts in place of Euler's ("Jamba — SSM-Transformer
 * Híbrido", section "Mamba-3: a linha de base de SSM puro em 2026", item 1: a more
 * expressive recurrence, a convolution-like operation on the state input inside the
 * recurrence; the key-terms rows "Exponential-trapezoidal discretization" of the zh and
 * hi lessons "Phase 10 · 21 Jamba hybrid SSM-Transformer": it subsumes Mamba-2's Euler
 * discretisation). No page gives a formula; the reading implemented is a two-point rule
 * on the step's input integral, the current input weighted lam_t and the older one
 * (decayed across the step) 1 - lam_t:
 *     h_t = exp(dt_t A) h_{t-1} + dt_t ((1 - lam_t) exp(dt_t A) B_{t-1} x_{t-1} + lam_t B_t x_t),
 * y_t as in ssm_scan_fwd. lam [batch, L, d_inner] (io dtype, laid out like dt) is the
 * weight per step and channel: 1 is Euler's step (ssm_scan_fwd's recurrence), 1/2 the
 * trapezoid rule; NULL = 1/2 everywhere. Any value is accepted; [0, 1] keeps both taps
 * non-negative. x_prev [batch, d_inner] and B_prev [batch, d_state] (io dtype) are the
 * input before step 0: NULL and NULL for a sequence with no earlier input; to resume a
 * sequence pass the last step's x and B of the previous part (with its h_final as h0).
 * Given together or not at all (else SSM_ERR_NULL). Other arguments, layouts, the
 * chunking (with the same decay-horizon bound) and the workspace
 * (ssm_scan_fwd_workspace_ex) are those of ssm_scan_fwd_ex. y must not overlap x, x_prev
 * or lam (SSM_ERR_UNSUPPORTED): a chunk's rescan reads the row before it. Alignment: as
 * ssm_scan_fwd_ex; x_prev and lam one element, B_prev 4 bytes.
 *
 * ssm_step_trap: one decode token of the same recurrence. x_prev [n_layers, n_seq,
 * d_inner] and B_prev [n_layers, n_seq, d_state] are the previous token's x_t and B_t
 * (NULL and NULL before the first token); the caller keeps them, the library keeps
 * only h. lam_t [n_layers, n_seq, d_inner] is the token's weight (NULL = 1/2).
 * Otherwise as ssm_step; B_prev is aligned like B_t, lam_t one element.
 * ssm_step_trap_replay is its one-thread-per-channel reference with the same fp32
 * operations in the same order: with lam = lam_t (or 1/2), wc = dt_t * lam,
 * wp = dt_t * (1 - lam), up = wp * x_prev, uc = wc * x_t, and per state n with
 * a = exp(dt_t A[n]),
 *     h[n] = fma(a, fma(up, B_prev[n], h[n]), uc * B_t[n]),
 * then the output as in ssm_step; the two agree bit for bit. */
ssm_status ssm_scan_fwd_trap(const void *x, const void *dt, const float *A, const void *B,
                             const void *C, const float *D, const void *z, const float *h0,
                             const void *x_prev, const void *B_prev, const void *lam, void *y,
                             float *h_final, int64_t batch, int64_t L, int64_t d_inner,
                             int32_t d_state, ssm_dtype io, int64_t chunk_len, void *workspace,
                             size_t workspace_bytes, void *hip_stream);
ssm_status ssm_step_trap(float *h, const void *x_prev, const void *B_prev, const void *x_t,
                         const void *dt_t, const void *lam_t, const float *A, const void *B_t,
                         const void *C_t, const float *D, const void *z_t, void *y_t,
                         int64_t n_layers, int64_t n_seq, int64_t d_inner, int32_t d_state,
                         ssm_dtype io, void *hip_stream);
ssm_status ssm_step_trap_replay(float *h, const void *x_prev, const void *B_prev,
                                const void *x_t, const void *dt_t, const void *lam_t,
                                const float *A, const void *B_t, const void *C_t, const float *D,
                                const void *z_t, void *y_t, int64_t n_layers, int64_t n_seq,
                                int64_t d_inner, int32_t d_state, ssm_dtype io,
                                void *hip_stream);

/* ------------------------------------------------------------------ MIMO projections
 * ssm_scan_fwd_mimo: the prefill with multi-input multi-output projections, the third
 * Mamba-3 item of "Jamba — SSM-Transformer Híbrido", section "Mamba-3: a linha de base
 * de SSM puro em 2026" (matrix-valued projections in place of scalar per-feature ones,
 * for more modelling power and better hardware use at inference without a longer
 * decode). The page gives no formula; the reading implemented: each channel takes
 * `rank` inputs and gives `rank` outputs, and B_t, C_t are d_state x rank matrices,
 *     h_t[n] = exp(dt_t A[n]) h_{t-1}[n] + dt_t sum_r B_t[n][r] x_t[r]
 *     y_t[r] = (sum_n C_t[n][r] h_t[n] + D x_t[r]) * silu(z_t[r])
 * The state is d_state per channel as in ssm_scan_fwd; rank = 1 is ssm_scan_fwd_ex.
 *   x, z, y : [batch, L, d_inner, rank] of io (rank fastest); dt: [batch, L, d_inner]
 *   B, C    : [batch, L, d_state, rank] of io;  A, D, h0, h_final as ssm_scan_fwd
 * rank is 1, 2, 4 or 8 (else SSM_ERR_UNSUPPORTED). x, z and y, and from rank 4 also
 * B and C, are aligned to min(16, rank * element size) bytes (else SSM_ERR_ALIGN);
 * other alignments, the chunking (with the same
 * decay-horizon bound, which does not depend on rank) and the errors are those of
 * ssm_scan_fwd_ex. The workspace comes from ssm_scan_fwd_mimo_workspace (0 for an
 * invalid shape or rank). y may be x itself but must not overlap it otherwise.
 * Arithmetic: the state is fp32 throughout. From rank 4 the sum over ranks for B_t x_t
 * is formed on the matrix cores (exact products, fp32 sums), and with bf16 io (and
 * d_state >= 4) so are the output sums over states, whose state operand is rounded to
 * bf16 (to nearest even): that adds at most 2^-8 sum_n |C[n][r] h[n]| to y[r], the
 * size of y's own rounding to bf16. With fp32 io the output sums are fp32 fused
 * multiply-adds, as in the decode.
 *
 * ssm_step_mimo: one decode token of the same recurrence for every (layer, sequence,
 * channel), h updated in place.
 *   h          : [n_layers, n_seq, d_inner, d_state] float32
 *   x_t, z_t, y_t : [n_layers, n_seq, d_inner, rank] of io;  dt_t: [n_layers, n_seq, d_inner]
 *   B_t, C_t   : [n_layers, n_seq, d_state, rank] of io (4-byte aligned)
 *   A, D       : as ssm_step
 * Per channel the fp32 operations are, in this order (up to rank 2 the same as the
 * prefill's, so L steps equal a one-chunk prefill, chunk_len = L, bit for bit; from
 * rank 4 the prefill forms its sums as described above):
 *   xd[r] = dt x[r];  for n ascending: u = B[n][0] xd[0], then u = fma(B[n][r], xd[r], u)
 *   for r = 1 .. rank-1; h[n] = fma(e2(dt (A[n] log2 e)), h[n], u);
 *   acc[r] = fma(C[n][r], h[n], acc[r]) (acc from 0);  y[r] = fma(D, x[r], acc[r]),
 *   gated y[r] * (z[r] * rcp(1 + e2(-z[r] log2 e))). */
size_t ssm_scan_fwd_mimo_workspace(int64_t batch, int64_t L, int64_t d_inner, int32_t d_state,
                                   int32_t rank, int64_t chunk_len);
ssm_status ssm_scan_fwd_mimo(const void *x, const void *dt, const float *A, const void *B,
                             const void *C, const float *D, const void *z, const float *h0,
                             void *y, float *h_final, int64_t batch, int64_t L, int64_t d_inner,
                             int32_t d_state, int32_t rank, ssm_dtype io, int64_t chunk_len,
                             void *workspace, size_t workspace_bytes, void *hip_stream);
ssm_status ssm_step_mimo(float *h, const void *x_t, const void *dt_t, const float *A,
                         const void *B_t, const void *C_t, const float *D, const void *z_t,
                         void *y_t, int64_t n_layers, int64_t n_seq, int64_t d_inner,
                         int32_t d_state, int32_t rank, ssm_dtype io, void *hip_stream);

/* ------------------------------------------------------------------ profiling
 * The same computation as ssm_scan_fwd_ex / ssm_scan_fwd_c64 / ssm_scan_fwd_fused /
 * ssm_scan_fwd_trap / ssm_scan_fwd_mimo, which additionally records four caller-created HIP events (hipEvent_t, passed
 * as void*) on hip_stream: events[0] before the chunk-summary kernel, events[1] after it,
 * events[2] after the carry-scan kernel, events[3] after the rescan kernel. With a
 * single chunk the first two phases launch nothing and their events are recorded
 * back to back. No work is skipped. n_events must be 4 (else SSM_ERR_NULL). For
 * benchmarks that time the kernels from inside the library's stream order. */
ssm_status ssm_scan_fwd_profiled(const void *x, const void *dt, const float *A, const void *B,
                                 const void *C, const float *D, const void *z, const float *h0,
                                 void *y, float *h_final,
                                 int64_t batch, int64_t L, int64_t d_inner, int32_t d_state,
                                 ssm_dtype io, int64_t chunk_len, void *workspace,
                                 size_t workspace_bytes, void *hip_stream,
                                 void *const *events, int32_t n_events);
ssm_status ssm_scan_fwd_c64_profiled(const void *x, const void *dt, const float *A,
                                     const void *B, const void *C, const float *D,
                                     const void *z, const float *h0, void *y, float *h_final,
                                     int64_t batch, int64_t L, int64_t d_inner, int32_t d_state,
                                     ssm_dtype io, int64_t chunk_len, void *workspace,
                                     size_t workspace_bytes, void *hip_stream,
                                     void *const *events, int32_t n_events);
ssm_status ssm_scan_fwd_fused_profiled(const void *x_in, const void *dt_raw, const float *A,
                                       const void *B, const void *C, const float *D,
                                       const void *z, const float *h0, const float *conv_w,
                                       const float *conv_b, int32_t conv_k,
                                       const void *conv_state0, void *conv_state_out,
                                       const float *dt_bias, void *y, float *h_final,
                                       int64_t batch, int64_t L, int64_t d_inner,
                                       int32_t d_state, ssm_dtype io, int64_t chunk_len,
                                       void *workspace, size_t workspace_bytes, void *hip_stream,
                                       void *const *events, int32_t n_events);

ssm_status ssm_scan_fwd_trap_profiled(const void *x, const void *dt, const float *A,
                                      const void *B, const void *C, const float *D,
                                      const void *z, const float *h0, const void *x_prev,
                                      const void *B_prev, const void *lam, void *y,
                                      float *h_final, int64_t batch, int64_t L, int64_t d_inner,
                                      int32_t d_state, ssm_dtype io, int64_t chunk_len,
                                      void *workspace, size_t workspace_bytes, void *hip_stream,
                                      void *const *events, int32_t n_events);
ssm_status ssm_scan_fwd_mimo_profiled(const void *x, const void *dt, const float *A,
                                      const void *B, const void *C, const float *D,
                                      const void *z, const float *h0, void *y, float *h_final,
                                      int64_t batch, int64_t L, int64_t d_inner, int32_t d_state,
                                      int32_t rank, ssm_dtype io, int64_t chunk_len,
                                      void *workspace, size_t workspace_bytes, void *hip_stream,
                                      void *const *events, int32_t n_events);

/* ------------------------------------------------------------------ misc */
const char *ssm_status_str(ssm_status s);   /* static string, never NULL */
const char *ssm_last_error(void);           /* this thread's last detail, "" if none */
int32_t ssm_abi_version(void);              /* 3 */

#ifdef __cplusplus
}
#endif
#endif /* SSM_SCAN_H */
