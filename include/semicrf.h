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
 *    shape supported (SEMICRF_ERR_UNSUPPORTED: C > 128; K above 8193 when C <= 7,
 *    2049 when C <= 16, 513 when C <= 64, and for 64 < C <= 128 whatever the 160 KB
 *    of LDS of a compute unit holds: 129 down to 97 at C = 128; semicrf_workspace_bytes
 *    returns 0 for such shapes).  A failed
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
    SEMICRF_ERR_DEVICE = 4,       /* a HIP launch or copy failed */
    SEMICRF_ERR_UNIMPLEMENTED = 5 /* reserved: no entry point of this library returns it */
} semicrf_status;

typedef enum {
    SEMICRF_OP_LOGZ = 0,
    SEMICRF_OP_BACKWARD = 1,
    SEMICRF_OP_VITERBI = 2,
    SEMICRF_OP_PREFIX = 3
} semicrf_op;

/* Human-readable name of a status code (static string, never NULL). */
const char* semicrf_status_string(int status);

/* Checkpoint interval for a padded length T and maximum duration K: delta if delta > 0,
 * else ceil(sqrt(T*K)) (EN explainer, "2. Methodology", "Checkpointing": an interval of
 * about sqrt(TK)); clamped to [1, T].  0 on bad input. */
int semicrf_checkpoint_interval(int T, int K, int delta);


/* The checkpoint interval `op` uses for delta = 0 (semicrf_viterbi takes none and always
 * uses it).  Every span is swept at once, so where the round kernels run (C <= 16,
 * K <= 1025) and for log Z and the backward everywhere, the interval is the one, over
 * every span count n (interval ceil(T/n)), that minimises
 * (interval + burn-in 3K) * ceil(workgroups / share): workgroups = B * spans for log Z, the
 * decode and a backward whose two directions share a workgroup (small label counts), else
 * twice that; share = 224 workgroups (7/8 of the MI355X's 256 compute units, leaving room
 * for a concurrent call) where the round kernels run, else 256.  Intervals shorter than
 * the burn-in are not taken (unless T is); ties go to the longer interval.  The decode
 * outside the round kernels takes ceil(sqrt(T*K)), halved when the batch holds at most
 * 128 spans of that length and each is at least four burn-ins (12 K) long.  0 on bad or
 * unsupported input. */
int semicrf_default_interval(semicrf_op op, int B, int T, int C, int K);

/* Bytes of workspace that `op` needs for these shapes (delta as the call takes it: > 0 an
 * explicit interval, 0 the default above).  0 if the arguments are invalid or
 * unsupported. */
size_t semicrf_workspace_bytes(semicrf_op op, int B, int T, int C, int K, int delta);

/* Centred prefix sums alone (EN explainer, "2. Methodology": "Emission Baseline
 * Centering" then "On-the-Fly Edge Computation via Prefix Sums"):
 *   S[b, 0, c] = 0,  S[b, t, c] = sum_{u < t} (em[b, u, c] - nu[b, c])  for t <= L_b,
 * nu[b, c] = mean of em[b, :L_b, c]; S[b, t, c] = S[b, L_b, c] for t > L_b.
 * Output: S [B, T+1, C] float64 (device).  Workspace: semicrf_workspace_bytes(
 * SEMICRF_OP_PREFIX, ...).  The other calls compute the same S internally. */
int semicrf_prefix(const float* emissions, const int32_t* lengths, int B, int T, int C,
                   hipStream_t stream, void* workspace, size_t workspace_bytes, double* S);

/* ------------------------------------------------------------------ the three calls
 * Each takes (emissions, lengths, trans, dur, sizes, stream) as the problem statement
 * gives them, plus a caller-owned workspace and the outputs. */

/* log Z for every sequence: the log-sum-exp of the scores of all segmentations
 * (EN explainer, "2. Methodology", "Streaming Forward-Backward with Ring Buffers",
 * forward pass).  delta: checkpoint interval (0 = semicrf_default_interval(SEMICRF_OP_LOGZ,
 * B, T, C, K)), the
 * same value as given to semicrf_workspace_bytes.  Output: log_z [B] float32. */
int semicrf_logz(const float* emissions, const int32_t* lengths, const float* trans,
                 const float* dur, int B, int T, int C, int K, int delta, hipStream_t stream,
                 void* workspace, size_t workspace_bytes, float* log_z);

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
 * delta: checkpoint interval (0 = semicrf_default_interval(SEMICRF_OP_BACKWARD, B, T, C,
 * K)); results do not
 * depend on it beyond rounding. */
int semicrf_backward(const float* emissions, const int32_t* lengths, const float* trans,
                     const float* dur, int B, int T, int C, int K, int delta,
                     hipStream_t stream, void* workspace, size_t workspace_bytes,
                     const float* grad_log_z, float* grad_emissions, float* grad_trans,
                     float* grad_dur, float* marginals, float* log_z);

/* Max-plus decode of the best segmentation (the Viterbi counterpart of the forward
 * pass).  Every max-plus step keeps the shortest segment, then the lowest previous
 * label, among equal candidates, and the decode ends at the lowest best final label.
 * When several segmentations share the best score (to fp32 rounding), the one returned
 * may differ from the one these rules give in exact arithmetic; a decision that beats
 * every alternative by more than rounding is always taken as in exact arithmetic.
 * Outputs:
 *   best_score [B]    float32  score of the best segmentation
 *   labels     [B, T] int32    label of every position, -1 at t >= lengths[b]
 *   seg_start  [B, T] uint8    1 where a segment starts, else 0 */
int semicrf_viterbi(const float* emissions, const int32_t* lengths, const float* trans,
                    const float* dur, int B, int T, int C, int K, hipStream_t stream,
                    void* workspace, size_t workspace_bytes, float* best_score,
                    int32_t* labels, uint8_t* seg_start);

/* ------------------------------------------------------------------ extended calls
 * The same three calls (and the training loss) with optional extras.  A NULL options
 * pointer, or a zero-initialised struct, gives exactly the plain call. */
typedef struct semicrf_options {
    /* Boundary projections (EN explainer, "2. Methodology", "Boundary Projections": start
     * and end features computed apart and added to the edge potential), inputs of every
     * call:
     *   proj_start [B, T, C] or NULL: score of a segment of label c that starts at t
     *   proj_end   [B, T, C] or NULL: score of a segment of label c whose last position is t
     * so a segment [s, e) of label c gains proj_start[b, s, c] + proj_end[b, e-1, c].  NULL
     * means zeros; values at t >= lengths[b] are ignored; the values must be finite (a
     * large negative value, e.g. -1e4, effectively forbids a start or end); not centred. */
    const float* proj_start;
    const float* proj_end;
    /* Backward and training-loss outputs, each optional (NULL):
     *   grad_proj_start [B, T, C]  g_b times the probability that a segment of label c
     *                              starts at t (d/d proj_start)
     *   grad_proj_end   [B, T, C]  g_b times the probability that a segment of label c has
     *                              its last position at t (d/d proj_end) */
    float* grad_proj_start;
    float* grad_proj_end;
    /* Backward outputs, each optional (NULL):
     *   boundary  [B, T]  probability that a segment starts at t (1 at t = 0; EN explainer,
     *                     "4. Results and Benchmarks": boundary probabilities)
     *   node_mass [B, T]  the sum over labels of the node marginals as the forward and
     *                     backward values give them, before the marginals are divided by
     *                     it: 1 in exact arithmetic, so |node_mass - 1| measures the
     *                     rounding of the streamed recurrences (0 at padding) */
    float* boundary;
    float* node_mass;
    /* Stage timing: NULL, or events created by the caller (hipEventCreate), one more than
     * the call's stage count; events[i] is recorded on `stream` when stage i begins and
     * the last when the call's work ends.  No synchronisation.
     *   logz:     0 centring + prefix scan, 1 forward sweep
     *   backward: 0 centring + prefix scan, 1 the checkpoint spans of both directions
     *             with their per-position values, 2 seam check and repair, 3 segment
     *             posteriors, 4 node marginals and gradient reductions
     *   viterbi:  0 centring + prefix scan, 1 max-plus checkpoint spans with the seam
     *             check, repair and final label, 2 backtrace */
    hipEvent_t* events;
    /* Checkpoint spans swept at once.  The sweeps are sequential in the position; every
     * span of delta positions is swept at the same time instead, starting 3K positions
     * early (at least 64) from a ring in which every entry is equal.  The values a span
     * then reaches equal the exact ones plus one constant, to within rounding; at each
     * checkpoint the library compares the two spans' ring values over the K positions
     * before it, takes the constant from them and accepts the seam when every entry is
     * within seam_tolerance of it (natural-log units; 0 = the default, 1e-4).  From the
     * first seam that is not accepted the sequence is swept again in order, exactly as a
     * single sweep would.
     *   seam_bound   [B] float32 or NULL: per sequence, the sum over both directions'
     *                accepted seams of the largest deviation from the constant; no value
     *                of the call moves by more than it (beyond rounding) from the values
     *                of sweeps run in order
     *   seam_repairs [B] int32 or NULL: the number of directions (0..2) swept again in
     *                order from a seam that was not accepted
     * A negative seam_tolerance accepts no seam (every sequence is swept in order after
     * its first span: the exact fallback, for testing). */
    float* seam_bound;
    int32_t* seam_repairs;
    double seam_tolerance;
} semicrf_options;

#define SEMICRF_LOGZ_STAGES 2
#define SEMICRF_BACKWARD_STAGES 5
#define SEMICRF_VITERBI_STAGES 3

int semicrf_logz_ex(const float* emissions, const int32_t* lengths, const float* trans,
                    const float* dur, int B, int T, int C, int K, int delta,
                    hipStream_t stream, void* workspace, size_t workspace_bytes, float* log_z,
                    const semicrf_options* options);
int semicrf_backward_ex(const float* emissions, const int32_t* lengths, const float* trans,
                        const float* dur, int B, int T, int C, int K, int delta,
                        hipStream_t stream, void* workspace, size_t workspace_bytes,
                        const float* grad_log_z, float* grad_emissions, float* grad_trans,
                        float* grad_dur, float* marginals, float* log_z,
                        const semicrf_options* options);
int semicrf_viterbi_ex(const float* emissions, const int32_t* lengths, const float* trans,
                       const float* dur, int B, int T, int C, int K, hipStream_t stream,
                       void* workspace, size_t workspace_bytes, float* best_score,
                       int32_t* labels, uint8_t* seg_start, const semicrf_options* options);

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
 * grad_emissions [B, T, C], grad_trans [C, C], grad_dur [K, C] and, through the options,
 * grad_proj_start / grad_proj_end [B, T, C] (expected minus gold feature counts; the
 * emission gradient includes the centring; 0 at padding).  Options: projections and
 * their gradients only (the other fields must be NULL).  A gold segmentation with a
 * segment longer than K, a label outside [0, C), a label change inside a segment or no
 * start at t = 0 gives NaN for that sequence and raises the status flag, like an invalid
 * length; its gold counts are then left out of the gradients, which keep only its log Z
 * half.  Workspace: semicrf_workspace_bytes(SEMICRF_OP_BACKWARD, ...). */
int semicrf_nll(const float* emissions, const int32_t* lengths, const float* trans,
                const float* dur, const int32_t* gold_labels, const uint8_t* gold_seg_start,
                int B, int T, int C, int K, int delta, hipStream_t stream, void* workspace,
                size_t workspace_bytes, const float* grad_nll, float* nll,
                float* grad_emissions, float* grad_trans, float* grad_dur,
                const semicrf_options* options);

/* ------------------------------------------------------------------ no allocation
 * For callers that cannot allocate device memory at all: code under HIP graph capture,
 * tight serving loops, harnesses that forbid hipMalloc.  semicrf_logz without a
 * workspace argument: the workspace is a static device array of
 * SEMICRF_STATIC_SCRATCH_BYTES inside the library, one per GPU, held from the first
 * call on that GPU until the process ends.  The call allocates nothing (no hipMalloc,
 * no allocating library routine).  Shapes whose semicrf_workspace_bytes(
 * SEMICRF_OP_LOGZ, ...) exceeds the array return SEMICRF_ERR_WORKSPACE before any
 * launch.  Every call on one GPU shares that GPU's array, so calls that overlap on one
 * GPU (on different streams, or from different threads) race and must be serialised
 * by the caller.  An invalid length gives NaN in log_z as for semicrf_logz; its status
 * flag is not readable.  The array lives on the device of `stream` (the current
 * device for the NULL stream). */
#define SEMICRF_STATIC_SCRATCH_BYTES ((size_t)32 << 20)
int semicrf_logz_static(const float* emissions, const int32_t* lengths, const float* trans,
                        const float* dur, int B, int T, int C, int K, int delta,
                        hipStream_t stream, float* log_z);

/* Synchronously reads the device status flag left in `workspace` by the last call
 * that used it (after waiting for `stream`).  SEMICRF_OK, SEMICRF_ERR_INVALID if a
 * length was outside [1, T], or SEMICRF_ERR_DEVICE if the copy failed. */
int semicrf_read_status(const void* workspace, hipStream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* SEMICRF_H */
