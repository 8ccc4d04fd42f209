/*
 * semicrf.h — C ABI of the MI355X (gfx950) streaming semi-Markov CRF library.
 *
 * Method: "Streaming Structured Inference with Flash-SemiCRF" (pages: thelatestinai
 * abstract card; gist.science explainers in English, Dutch and Chinese).  A semi-CRF
 * labels whole segments [s, s+k), 1 <= k <= K, with one of C labels.  The potential
 * of a segment of label c that follows a segment of label c' is
 *
 *     S[s+k, c] - S[s, c] + dur[k-1, c] + trans[c', c]
 *
 * where S is the prefix sum of the emissions after subtracting their per-sequence,
 * per-label mean (EN explainer, "2. Methodology": "On-the-Fly Edge Computation via
 * Prefix Sums" and "Emission Baseline Centering").  The first segment of a sequence
 * pays no transition score and nothing is paid after the last one.  The library
 * evaluates every potential on the fly from S; the T*K*C^2 edge tensor is never
 * stored (EN explainer, "1. Problem Statement").
 *
 * Conventions shared by every entry point
 *  - All array arguments are DEVICE pointers to dense row-major arrays with the
 *    label index innermost:
 *        emissions [B, T, C] float32     lengths [B] int32 (1 <= lengths[b] <= T)
 *        trans     [C, C]    float32     (row = previous label, column = next label)
 *        dur       [K, C]    float32     (row k-1 scores a segment of length k)
 *    Emissions at t >= lengths[b] are ignored.  -inf in trans or dur forbids the
 *    transition / duration.
 *  - Ownership: the caller allocates and frees every input, output and the
 *    workspace.  The library allocates no device memory and keeps no pointer or
 *    other state after a call returns.  Calls on different streams with distinct
 *    workspaces may run concurrently.
 *  - Execution: all work is enqueued on `stream`; no call synchronises the host.
 *    Outputs are valid once the stream reaches that point.  Results are bitwise
 *    reproducible for the same inputs, shapes and checkpoint interval (fixed-order
 *    reductions, no floating-point atomics).
 *  - Errors: every call returns a semicrf_status and never aborts.  Host-side
 *    checks: B, T, C, K >= 1, required pointers non-NULL, workspace large enough,
 *    shape supported (SEMICRF_ERR_UNSUPPORTED: C > 128; K above 2049 when C <= 7,
 *    1025 when C = 8, 513 when C <= 16, 257 when C <= 64, and for 64 < C <= 128
 *    whatever the 160 KB of LDS of a compute unit holds: 129 down to 97 at C = 128;
 *    semicrf_workspace_bytes returns 0 for such shapes).  A failed
 *    kernel launch returns SEMICRF_ERR_DEVICE.  A length outside [1, T] is only
 *    visible on the device: that sequence is processed as if clamped to [1, T],
 *    its log Z / Viterbi score is set to NaN, and a flag is raised in the
 *    workspace that semicrf_read_status() returns.
 *  - Workspace: at least semicrf_workspace_bytes(op, ...) bytes of device memory,
 *    256-byte aligned, passed to the call of that op.  Its contents on entry do not
 *    matter and are overwritten.
 */
#ifndef SEMICRF_H
#define SEMICRF_H

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    SEMICRF_OK = 0,
    SEMICRF_ERR_INVALID = 1,      /* bad scalar argument or NULL pointer, or a device-flagged length */
    SEMICRF_ERR_WORKSPACE = 2,    /* workspace NULL, too small or misaligned */
    SEMICRF_ERR_UNSUPPORTED = 3,  /* shape outside the supported range */
    SEMICRF_ERR_DEVICE = 4        /* a HIP launch or copy failed */
} semicrf_status;

typedef enum {
    SEMICRF_OP_LOGZ = 0,
    SEMICRF_OP_BACKWARD = 1,
    SEMICRF_OP_VITERBI = 2,
    SEMICRF_OP_PREFIX = 3
} semicrf_op;

/* Human-readable name of a status code (static string, never NULL). */
const char* semicrf_status_string(int status);

/* Checkpoint interval used by semicrf_backward for a padded length T and maximum
 * duration K: delta if delta > 0, else ceil(sqrt(T*K)) (EN explainer, "2. Methodology",
 * "Checkpointing": interval of about sqrt(TK)); clamped to [1, T].  0 on bad input. */
int semicrf_checkpoint_interval(int T, int K, int delta);

/* Bytes of workspace that `op` needs for these shapes (delta as above; ignored by
 * LOGZ and VITERBI).  0 if the arguments are invalid or unsupported. */
size_t semicrf_workspace_bytes(int op, int B, int T, int C, int K, int delta);

/* Centred prefix sums alone (EN explainer, "2. Methodology": "Emission Baseline
 * Centering" then "On-the-Fly Edge Computation via Prefix Sums"):
 *   S[b, 0, c] = 0,  S[b, t, c] = sum_{u < t} (em[b, u, c] - nu[b, c])  for t <= L_b,
 * nu[b, c] = mean of em[b, :L_b, c]; S[b, t, c] = S[b, L_b, c] for t > L_b.
 * Output: S [B, T+1, C] float64 (device).  Workspace: semicrf_workspace_bytes(
 * SEMICRF_OP_PREFIX, ...).  The other calls compute the same S internally. */
int semicrf_prefix(const float* emissions, const int32_t* lengths, int B, int T, int C,
                   hipStream_t stream, void* workspace, size_t workspace_bytes, double* S);

/* Boundary projections (EN explainer, "2. Methodology", "Boundary Projections": start
 * and end features computed apart and added to the edge potential).  Every call below
 * that takes them accepts
 *   proj_start [B, T, C] float32 or NULL  score of a segment of label c that starts at t
 *   proj_end   [B, T, C] float32 or NULL  score of a segment of label c whose last
 *                                         position is t
 * so a segment [s, e) of label c gains proj_start[b, s, c] + proj_end[b, e-1, c].  NULL
 * means zeros; values at t >= lengths[b] are ignored; the values must be finite (a large
 * negative value, e.g. -1e4, effectively forbids a start or end).  They are not centred. */

/* log Z for every sequence: the log-sum-exp of the scores of all segmentations
 * (EN explainer, "2. Methodology", "Streaming Forward-Backward with Ring Buffers",
 * forward pass).  Output: log_z [B] float32. */
int semicrf_logz(const float* emissions, const int32_t* lengths, const float* trans,
                 const float* dur, const float* proj_start, const float* proj_end, int B,
                 int T, int C, int K, hipStream_t stream, void* workspace,
                 size_t workspace_bytes, float* log_z);

/* Exact gradients of sum_b grad_log_z[b] * log Z_b (EN explainer, "2. Methodology",
 * backward pass with recomputation from checkpoints every `delta` positions;
 * "4. Results and Benchmarks": exact gradients).  Inputs as above plus
 *   grad_log_z [B] float32, or NULL for all ones.
 * Outputs (all overwritten; padding positions t >= lengths[b] are set to 0):
 *   grad_emissions [B, T, C] float32  d/d emissions, including the centring mean
 *   grad_trans     [C, C]    float32  summed over the batch
 *   grad_dur       [K, C]    float32  summed over the batch
 *   marginals      [B, T, C] float32  or NULL: posterior probability that position t
 *                                     lies in a segment of label c (sums to 1 over c)
 *   log_z          [B]       float32  or NULL
 *   grad_proj_start [B, T, C] float32 or NULL: d/d proj_start, g_b times the probability
 *                                     that a segment of label c starts at t
 *   grad_proj_end   [B, T, C] float32 or NULL: d/d proj_end, g_b times the probability
 *                                     that a segment of label c has its last position at t
 *   boundary       [B, T]    float32  or NULL: probability that a segment starts at t
 *                                     (1 at t = 0; EN explainer, "4. Results and
 *                                     Benchmarks": boundary probabilities)
 * delta: checkpoint interval (0 = ceil(sqrt(T*K))); results do not depend on it
 * beyond rounding. */
int semicrf_backward(const float* emissions, const int32_t* lengths, const float* trans,
                     const float* dur, const float* proj_start, const float* proj_end, int B,
                     int T, int C, int K, int delta, hipStream_t stream, void* workspace,
                     size_t workspace_bytes, const float* grad_log_z, float* grad_emissions,
                     float* grad_trans, float* grad_dur, float* marginals, float* log_z,
                     float* grad_proj_start, float* grad_proj_end, float* boundary);

/* Training loss of gold segmentations and its gradients.  nll[b] = log Z_b - score_b(y*),
 * the negative log-probability of the gold segmentation y* (the training loss of the
 * pages' convergence check, EN explainer, "4. Results and Benchmarks"); score sums, over
 * the gold segments [s, e) of label c, S[e,c] - S[s,c] + dur[e-s-1, c] (+ the
 * projections) and, between consecutive segments, trans[c', c] (the same centred
 * potential as log Z, "2. Methodology").  Inputs as semicrf_backward plus
 *   gold_labels    [B, T] int32  label of every position t < lengths[b]
 *   gold_seg_start [B, T] uint8  1 at each gold segment's first position (t = 0 must be 1)
 *   grad_nll       [B] float32 or NULL for all ones
 * Outputs: nll [B] float32, and the gradients of sum_b grad_nll[b] * nll[b] in
 * grad_emissions [B, T, C], grad_trans [C, C], grad_dur [K, C] and, each optional (NULL),
 * grad_proj_start / grad_proj_end [B, T, C] (expected minus gold feature counts; the
 * emission gradient includes the centring; 0 at padding).  A gold segmentation
 * with a segment longer than K, a label outside [0, C), a label change inside a segment or
 * no start at t = 0 gives NaN for that sequence and raises the status flag, like an
 * invalid length; its gold counts are then left out of the gradients, which keep only
 * its log Z half.  Workspace: semicrf_workspace_bytes(SEMICRF_OP_BACKWARD, ...). */
int semicrf_nll(const float* emissions, const int32_t* lengths, const float* trans,
                const float* dur, const float* proj_start, const float* proj_end,
                const int32_t* gold_labels, const uint8_t* gold_seg_start, int B, int T, int C,
                int K, int delta, hipStream_t stream, void* workspace, size_t workspace_bytes,
                const float* grad_nll, float* nll, float* grad_emissions, float* grad_trans,
                float* grad_dur, float* grad_proj_start, float* grad_proj_end);

/* Max-plus decode of the best segmentation (the Viterbi counterpart of the forward
 * pass).  Each max-plus step breaks ties toward the shortest segment, then the lowest
 * previous label.  For C <= 16 the forward sweep and a sweep over the mirrored sequence
 * meet in the middle and the best boundary of the meeting window joins them (lowest
 * position, then labels, on ties); for C > 16 one forward sweep ends at the lowest best
 * final label.  When several segmentations share the best score (to fp32 rounding),
 * which one is returned is therefore implementation-defined; a best segmentation that
 * beats every other by more than rounding is returned exactly.  Outputs:
 *   best_score [B]    float32  score of the best segmentation
 *   labels     [B, T] int32    label of every position, -1 at t >= lengths[b]
 *   seg_start  [B, T] uint8    1 where a segment starts, else 0 */
int semicrf_viterbi(const float* emissions, const int32_t* lengths, const float* trans,
                    const float* dur, const float* proj_start, const float* proj_end, int B,
                    int T, int C, int K, hipStream_t stream, void* workspace,
                    size_t workspace_bytes, float* best_score, int32_t* labels,
                    uint8_t* seg_start);

/* Stage-timed variants, for profiling.  Identical results to the calls above; in
 * addition, events[i] (created by the caller with hipEventCreate) is recorded on
 * `stream` when stage i begins, and events[NSTAGES] when the call's work ends, so
 * hipEventElapsedTime(events[i], events[i+1]) is the device time of stage i.
 * events must be non-NULL (else SEMICRF_ERR_INVALID).  No synchronisation.
 *   logz:     0 centring + prefix scan, 1 forward sweep
 *   backward: 0 centring + prefix scan, 1 checkpoint sweeps (both directions at once;
 *             empty when delta >= T), 2 span recompute, 3 segment posteriors,
 *             4 node marginals and gradient reductions
 *   viterbi:  0 centring + prefix scan, 1 max-plus sweep, 2 combine and backtrace */
#define SEMICRF_LOGZ_STAGES 2
#define SEMICRF_BACKWARD_STAGES 5
#define SEMICRF_VITERBI_STAGES 3
int semicrf_logz_staged(const float* emissions, const int32_t* lengths, const float* trans,
                        const float* dur, const float* proj_start, const float* proj_end, int B,
                        int T, int C, int K, hipStream_t stream, void* workspace,
                        size_t workspace_bytes, float* log_z, hipEvent_t* events);
int semicrf_backward_staged(const float* emissions, const int32_t* lengths, const float* trans,
                            const float* dur, const float* proj_start, const float* proj_end,
                            int B, int T, int C, int K, int delta, hipStream_t stream,
                            void* workspace, size_t workspace_bytes, const float* grad_log_z,
                            float* grad_emissions, float* grad_trans, float* grad_dur,
                            float* marginals, float* log_z, float* grad_proj_start,
                            float* grad_proj_end, float* boundary, hipEvent_t* events);
int semicrf_viterbi_staged(const float* emissions, const int32_t* lengths, const float* trans,
                           const float* dur, const float* proj_start, const float* proj_end,
                           int B, int T, int C, int K, hipStream_t stream, void* workspace,
                           size_t workspace_bytes, float* best_score, int32_t* labels,
                           uint8_t* seg_start, hipEvent_t* events);

/* Synchronously reads the device status flag left in `workspace` by the last call
 * that used it (after waiting for `stream`).  SEMICRF_OK, SEMICRF_ERR_INVALID if a
 * length was outside [1, T], or SEMICRF_ERR_DEVICE if the copy failed. */
int semicrf_read_status(const void* workspace, hipStream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* SEMICRF_H */
