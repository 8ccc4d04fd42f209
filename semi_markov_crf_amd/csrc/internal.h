// Internal interfaces between the C ABI (api.cpp) and the kernel translation units.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace semicrf {

// ------------------------------------------------------------------ problem shape
struct Shape {
    int B, T, C, K;
};

// Positions per tile of the emission reduction / prefix-scan kernels.
int scan_tile(int C);
// Positions per tile of the marginal and node-marginal kernels, and durations per chunk
// of the marginal kernel.
int marg_tile(int C, int K);
int marg_labels(int C);   // labels a k_marginals workgroup takes (a label group)
int marg_kchunk(int C, int K);

// ------------------------------------------------------------------ sweep configuration
// Lanes are grouped G per label; each lane covers KPL durations and CPL previous labels.
// ring layout bits: each position stored twice, RS apart (contiguous windows); E = 2^R
// ring for the linear-space bulk sum of the log-semiring sweep
enum { SWEEP_MIRRORED = 1, SWEEP_LINEAR = 2 };

struct SweepLds {
    int layout;          // SWEEP_MIRRORED | SWEEP_LINEAR bits
    int P;               // ring row pitch (floats)
    int CH;              // positions per staged chunk of S
    size_t bytes;        // dynamic LDS per workgroup (0: does not fit)
};

// Long-duration sweeps (sweep_xk.h): one chain wavefront and G bulk lanes per label, each
// lane holding kpl duration weights (a multiple of XK_UNROLL, at most the instance's
// kplmax), the rings of RS >= K + 2 slots per label in LDS, mirrored in LDS, or in a global
// scratch slice per workgroup (XK_RING_*).
constexpr int XK_UNROLL = 8;
// positions between base moves: entries written between two moves drift from their base
// by up to XK_REBASE times the per-position growth of the log partition function, and
// their fp32 rounding grows with that offset (8 positions: node-mass deviation about 3e-5
// at T = 6000, K = 1030, three times that with 16)
constexpr int XK_LOG_REBASE = 3;
constexpr int XK_REBASE = 1 << XK_LOG_REBASE;
constexpr int XK_PF = 2;           // staged S values per bulk lane and chunk
constexpr int XK_FROM = 1026;      // durations from which the long-duration sweeps run

// where the rings of the long-duration sweeps live (sweep_xk.h)
enum { XK_RING_LDS = 0, XK_RING_MIRRORED = 1, XK_RING_GLOBAL = 2 };
// rings of C * RS floats a workgroup keeps in global memory: the log ring (both semirings)
// unless it is in LDS, and the linear ring of the log semiring in the plain global layout
constexpr int xk_global_rings(bool maxp, int ring) {
    return ring == XK_RING_GLOBAL ? (maxp ? 1 : 2) : ring == XK_RING_MIRRORED ? (maxp ? 0 : 1) : 0;
}

struct XkCfg {
    bool ok;
    int G, kplmax, NT, kpl, RS, CH;
    int NE;              // log semiring: epochs of XK_REBASE positions in the shift table
    int ring;            // XK_RING_*
    size_t lds;          // dynamic LDS per workgroup
};
// per-launch parameters of the long-duration sweeps
struct XkParams {
    float* ring;         // [workgroups][rings held in global memory][C][RS], or NULL
    int RS, CH, kpl, NE;
};
// maxp: the max-plus sweep (one ring) instead of the log-semiring sweep (two)
XkCfg choose_xk(int C, int K, bool maxp);

struct SweepCfg {
    int G, KPL, CPL, GT; // instantiated kernel shape (KPL: register capacity per lane)
    int kpl;             // durations k >= 3 per lane actually used
    int BPL;             // round kernels: ring blocks of ROUND positions per bulk lane
    int CPr;             // round kernels: labels the chain wavefront broadcasts (>= C)
    int NT;              // threads per workgroup of the log-semiring sweep (multiple of 64)
    int NTv;             // threads per workgroup of the max-plus sweep
    bool split;          // log-semiring sweep by role, ROUND positions per barrier (C <= 16)
    int RS;              // ring slots per copy (power of two)
    SweepLds lse;        // log-semiring sweep
    SweepLds vit;        // max-plus sweep
    bool xk;             // the long-duration sweeps run (xk_lse, xk_vit) instead
    XkCfg xk_lse, xk_vit;
    bool ok;
};
SweepCfg choose_sweep(int C, int K);

// S rows staged per LDS chunk (at most): log-semiring sweep (plus one look-ahead row),
// max-plus sweep
__host__ __device__ constexpr int lse_chunk_max(int G) { return G >= 16 ? 64 : 16; }
constexpr int MAXPLUS_CHUNK_MAX = 64;

// Dynamic LDS of the log-semiring sweep: end-side and start-side S chunks [2][2][CH+1][C]
// + S(L) [C] (fp64), then the R ring (and the E ring when linear) [C+1][P], messages p and
// u [2][UP] each, and a per-thread sink [NT] (fp32).
inline size_t lse_lds_bytes(int C, int NT, int UP, int P, int CH, bool lin) {
    return (size_t)(4 * (CH + 1) * C + C) * 8 +
           (size_t)((lin ? 2 : 1) * (C + 1) * P + 4 * UP + NT) * 4;
}
// The round kernels (C <= 16): ROUND positions per workgroup barrier.
constexpr int ROUND = 4;
// Dynamic LDS of the log-semiring round kernel: S chunks [2][C][CH] and S(L) (fp64), the
// chunks' per-position factors [2][5 with projections, else 3][C][CH], the rings [C+1][P]
// (two when linear), bulk sums [2][CP][2][ROUND], staged ring entries [2][CP+1][2][ROUND],
// rebase shifts and dmax [CP rounded to 4], a sink and two constant blocks [16], staged
// message sums [2][CP][ROUND] and replay flags [4] (fp32), staged bases [2][CP] (fp64).
__host__ __device__ inline size_t lse_round_lds_bytes(int C, int CP, int P, int CH, bool lin,
                                                      bool proj) {
    const int cp4 = (CP + 3) / 4 * 4;
    return (size_t)(2 * CH * C + (C + 1) / 2 * 2) * 8 +
           (size_t)((proj ? 10 : 6) * C * CH + (lin ? 2 : 1) * (C + 1) * P + 4 * CP * ROUND +
                    4 * (CP + 1) * ROUND + 2 * cp4 + 16 + 2 * CP * ROUND + 4) * 4 +
           (size_t)2 * CP * 8;
}
// One direction's LDS region of the round kernel (16-byte aligned, so that the region of
// the second direction, when both share a workgroup, keeps every alignment).
__host__ __device__ inline size_t lse_round_region_bytes(int C, int CP, int P, int CH, bool lin,
                                                         bool proj) {
    return (lse_round_lds_bytes(C, CP, P, CH, lin, proj) + 15) / 16 * 16;
}
// Dynamic LDS of the max-plus round kernel (C <= 16): S chunks [2][C][CH] (fp64),
// with projections the chunks' end-side and start-side projections [2][2][C][CH], the
// ring [C+1][P], bulk maxima and their k [2][CP][2][ROUND], rebase shifts [CP rounded to
// 4], a sink and a constant block [12] (fp32).
inline size_t maxplus_round_lds_bytes(int C, int CP, int P, int CH, bool proj) {
    const int cp4 = (CP + 3) / 4 * 4;
    return (size_t)(2 * CH * C) * 8 +
           (size_t)((proj ? 4 : 0) * C * CH + (C + 1) * P + 4 * CP * ROUND + cp4 + 12) * 4;
}
// Dynamic LDS of the max-plus sweep: end-side and start-side S chunks [2][2][CH][C]
// (fp64), R ring [C+1][P] and u [2][UP] (fp32).
inline size_t maxplus_lds_bytes(int C, int UP, int P, int CH) {
    return (size_t)(4 * CH * C) * 8 + (size_t)((C + 1) * P + 2 * UP) * 4;
}

// MODE_SPEC: one workgroup per (span, sequence, direction), all at once: a span other than the first
//            starts `warm` positions early from a uniform ring (every entry equal) instead
//            of a checkpoint; its values then equal the exact ones up to a constant, to
//            within the rounding of the sweep, which the seam check verifies.  It writes its
//            outputs in its own frame, the ring values of the K positions that end its
//            burn-in (head) and its span (tail), and a checkpoint at its end.
// MODE_REPAIR: one per (sequence, direction): where a seam check failed, the sequence is
//            swept again from the checkpoint at the first failed seam to its end.
enum SweepMode { MODE_SPEC = 2, MODE_REPAIR = 3 };

struct SweepArgs {
    const double* S;        // [B][T+1][C] centred prefix sums
    const int* Leff;        // [B] clamped length, negated when the input length was invalid
    const float* trans;     // [C][C]
    const float* dur;       // [K][C]
    int B, T, C, K;
    int mode;               // MODE_SPEC: grid (nspans, B, ndir); MODE_REPAIR: grid (B, ndir)
    int delta;              // checkpoint interval
    int nspans;             // max spans per sequence (ceil(T / delta))
    int write_xa;           // write the per-position values X
    // checkpoints at span ends [2 dirs][B][nspans][...]; index 0 of the span axis is unused
    float* ck_ring;         // [..][K][C]
    double* ck_base;        // [..][C]
    float* ck_mprev;        // [..][C]
    double* ck_href;        // [..]
    // per-position outputs, natural-log units, [B][T+1][C]: the messages before the
    // transition step (X on (tout, t1] of a span)
    double* XF;             // forward: alpha[t, c]
    double* XB;             // backward: beta_bar[s, c]
    double* logz;           // [B] forward log Z
    double* logz_b;         // [B] log Z from the backward sweep (consistency check)
    // speculative spans (MODE_SPEC) and their repair (MODE_REPAIR)
    int warm;               // burn-in positions before a span
    double* head;           // [2 dirs][B][nspans][K][C] ring values (natural log, the
    double* tail;           //   span's own frame) of positions t0-K+1 .. t0 / t1-K+1 .. t1
    double* lzloc;          // [2 dirs][B] log Z of the last span, in its own frame
    const int* first_bad;   // [2 dirs][B] first span whose seam failed (nspans: none)
    const double* off;      // [2 dirs][B][nspans] frame offsets (natural log)
    // Viterbi
    uint32_t* bp;           // [B][T+1][C]: (k) | (previous label << 16)
    double* vfin;           // [B][C] values V(L, c) of the span that holds L, in its frame
};

// What the launchers receive: the kernels' arguments plus the boundary projections, which
// the kernels take as separate trailing arguments.  Projections are [B][T][C] or NULL
// (zeros): a segment [s, e) of label c gains proj_start[s, c] + proj_end[e-1, c].  Sweep
// position p of direction 0 adds proj_end[p-1] to the messages that end there and
// proj_start[p] to the ring entries that start there; on the mirrored sequence the two
// swap roles (proj_start[L-p] at the end side, proj_end[L-1-p] at the start side).
struct SweepLaunch : SweepArgs {
    const float* proj_start = nullptr;
    const float* proj_end = nullptr;
    float* xk_ring = nullptr;       // long-duration sweeps: the global ring scratch
};

// log-semiring sweep: grid (nspans, B, ndir) in MODE_SPEC, (B, ndir) in MODE_REPAIR;
// dispatches on cfg.lse.layout to the per-layout translation units
hipError_t launch_lse(const SweepCfg& cfg, const SweepLaunch& a, int ndir, hipStream_t stream);
hipError_t launch_lse_mirror(const SweepCfg& cfg, const SweepLaunch& a, int ndir, hipStream_t stream);
hipError_t launch_lse_plain(const SweepCfg& cfg, const SweepLaunch& a, int ndir, hipStream_t stream);
hipError_t launch_lse_log(const SweepCfg& cfg, const SweepLaunch& a, int ndir, hipStream_t stream);
// round kernels (C <= 16) with boundary projections
hipError_t launch_lse_round_proj(const SweepCfg& cfg, const SweepLaunch& a, int ndir, bool lin,
                                 hipStream_t stream);
hipError_t launch_maxplus_round_proj(const SweepCfg& cfg, const SweepLaunch& a, hipStream_t stream);
// max-plus sweep (Viterbi), forward only: grid (nspans, B) in MODE_SPEC, (B) in
// MODE_REPAIR; dispatches on cfg.vit.layout
hipError_t launch_maxplus(const SweepCfg& cfg, const SweepLaunch& a, hipStream_t stream);
hipError_t launch_maxplus_mirror(const SweepCfg& cfg, const SweepLaunch& a, hipStream_t stream);
hipError_t launch_maxplus_plain(const SweepCfg& cfg, const SweepLaunch& a, hipStream_t stream);
// long-duration sweeps (cfg.xk): same grids and modes
hipError_t launch_xk_lse(const XkCfg& xc, const SweepLaunch& a, int ndir, hipStream_t stream);
hipError_t launch_xk_maxplus(const XkCfg& xc, const SweepLaunch& a, hipStream_t stream);
// float words of the global ring scratch of the long-duration sweeps (0 in LDS)
size_t xk_ring_floats(const XkCfg& xc, int C, int workgroups, bool maxp);

// ------------------------------------------------------------------ seam check
struct SeamArgs {
    const double* head;     // [ndir][B][nspans][K][C] (see SweepArgs)
    const double* tail;
    const double* lzloc;    // [ndir][B]
    const int* Leff;        // [B]
    int B, C, K, delta, nspans;
    double tol;             // accepted half-range of tail - head (natural log); < 0: none
    double* off;            // [ndir][B][nspans] frame offsets (out)
    int* first_bad;         // [ndir][B] first failed seam, nspans if none (out)
    double* logz;           // [B] direction 0 (out, where no seam failed)
    double* logz_b;         // [B] direction 1 (out, where no seam failed)
    double* diag;           // [ndir][B][4]: sum and max of the accepted half-ranges, first
                            //   failed seam (-1: none), number of seams (out)
    double* stats;          // [ndir][B][nspans][3] scratch: max d, min d, finiteness mismatch
};
hipError_t launch_seam(const SeamArgs& s, int ndir, hipStream_t stream);
// bound [B] / repairs [B] (either may be NULL) from the seam check's diag
hipError_t launch_seam_report(const double* diag, int B, int ndir, float* bound, int* repairs,
                              hipStream_t stream);
// burn-in length of a speculative span and the default seam tolerance (natural log)
int spec_warm(int K);
constexpr double SEAM_TOL = 1.0e-4;

// ------------------------------------------------------------------ scans
// Per-tile column sums of the valid emissions; also writes the clamped lengths Leff
// (negated where the input length was outside [1, T]).
hipError_t launch_em_tile_sums(const float* em, const int32_t* lengths, int B, int T, int C,
                               double* tile_sums, int* Leff, hipStream_t stream);
// For each b: exclusive prefix (or suffix when reverse) over tiles of [B][n][C] doubles,
// written to `offsets`, and the totals to `totals` [B][C] (either may be NULL).
hipError_t launch_tile_scan(const double* tile_sums, int B, int n, int C, bool reverse,
                            double* offsets, double* totals, hipStream_t stream);
// Centred prefix sums S [B][T+1][C] from the emissions and the tile offsets / totals;
// status[0] = 1 if any length was invalid, else 0.
hipError_t launch_prefix(const float* em, const int* Leff, int B, int T, int C,
                         const double* tile_offsets, const double* totals, double* S, int* status,
                         hipStream_t stream);

// ------------------------------------------------------------------ marginals / gradients
// The transition step of every position, in place: XF / XB (the sweeps' messages before
// it) become AF / AB in base 2 (frame offsets added, log Z and S[L] folded in; see
// marginals.hip), and the transition posteriors are summed per tile group.
struct TransStepArgs {
    const double* S;
    const int* Leff;
    const float* trans;
    int B, T, C;
    int tile, ntiles, tpg, ngroups;   // as k_marginals
    double* XF;                       // [B][T+1][C], in: alpha, out: AF
    double* XB;                       // [B][T+1][C], in: beta_bar, out: AB
    const float* proj_start;          // [B][T][C] or NULL
    const float* proj_end;            // [B][T][C] or NULL
    const double* logz;
    // frame offsets of the speculative spans, [2 dirs][B][nspans] (NULL: none): added to
    // XF of forward span floor((s-1)/delta) and to XB of the mirrored span of L - s - 1
    const double* off;
    int delta, nspans;
    double* part_trans;               // [B][ngroups][C][C]
};
hipError_t launch_trans_step(const TransStepArgs& a, hipStream_t stream);

struct MargArgs {
    const double* S;
    const int* Leff;
    const float* dur;
    int B, T, C, K;
    int tile;               // positions per tile
    int kchunk;             // durations per staged chunk
    int ntiles;             // ceil((T+1) / tile)
    int tpg, ngroups;       // tiles per group of the duration / transition partials
    const double* AF;       // [B][T+1][C] from k_trans_step
    const double* AB;       // [B][T+1][C] from k_trans_step
    // [B][T][C]: inclusive prefix sum, inside each tile, of (start mass - end mass) of
    // the segments at each position (fp64 sums rounded once); the marginals' buffer, which
    // k_node_marginals turns into mu in place
    float* Dloc;
    double* dn_tile;        // [B][ntiles][C]: tile sums of (start mass - end mass)
    double* part_dur;       // [B][ngroups][K][C]: sums over a group's tiles
    float* pstart;          // [B][T][C] or NULL: raw start mass of segments at each position
    float* pend;            // [B][T][C] or NULL: raw mass of segments whose last position it is
    float* pbsum;           // [B][T] or NULL: raw start mass summed over labels
    int cg;                 // labels per label group (marg_labels(C))
    // [groups][B][T]: each label group's share of pbsum when there are several (NULL
    // otherwise); k_node_marginals adds them up in group order
    float* pb_part;
};
hipError_t launch_marginals(const MargArgs& a, hipStream_t stream);
// tiles per group of the posterior partials: enough groups to fill the device, the
// partials (B * groups * (K + C) * C doubles) within a fixed budget
int marg_tiles_per_group(int B, int ntiles, int C, int K);

// mu = tile offset + in-tile prefix Dloc, normalised per position; writes marginals, per-tile
// sums of mu and the per-tile mean normaliser.  The three boundary outputs hold the raw
// masses k_marginals wrote into them (start [B][T][C], end [B][T][C], start summed over
// labels [B][T]) and are rescaled in place: the boundary probability, and g times the
// normalised start and end marginals (any of them may be NULL).
struct BoundaryOut {
    const float* grad_log_z;
    float* grad_proj_start;
    float* grad_proj_end;
    float* boundary;
    float* node_mass;           // [B][T] or NULL: the per-position normaliser itself
    const float* pb_part;       // [npb][B][T] label groups' raw boundary sums, or NULL
    int npb;                    // (then boundary holds nothing yet)
};
hipError_t launch_node_marginals(const float* Dloc, const double* dn_off, const int* Leff,
                                 int B, int T, int C, int tile, int ntiles, float* mu,
                                 double* mu_tile, double* z_tile, const BoundaryOut& bo,
                                 hipStream_t stream);
hipError_t launch_grad_em(const float* mu, const double* mu_tot, const int* Leff,
                          const float* grad_log_z, int B, int T, int C, float* grad_em,
                          hipStream_t stream);
// scratch: reduce_scratch_doubles(C, K) doubles
size_t reduce_scratch_doubles(int C, int K);
hipError_t launch_reduce_partials(const double* part_dur, const double* part_trans,
                                  const double* z_tile, const int* Leff, const float* grad_log_z,
                                  int B, int C, int K, int tile, int ntiles, int tpg,
                                  double* scratch, float* grad_dur, float* grad_trans,
                                  hipStream_t stream);
hipError_t launch_write_logz(const double* logz, int B, float* out, hipStream_t stream);

// ------------------------------------------------------------------ gold-segmentation loss
struct GoldArgs {
    const double* S;            // [B][T+1][C] centred prefix sums
    const int* Leff;            // [B]
    const float* trans;         // [C][C]
    const float* dur;           // [K][C]
    const float* proj_start;    // [B][T][C] or NULL
    const float* proj_end;      // [B][T][C] or NULL
    const int32_t* labels;      // [B][T] gold label per position
    const uint8_t* seg_start;   // [B][T] 1 at each gold segment's first position
    int B, T, C, K;
    const double* logz;         // [B] from the backward pass
    const float* grad_nll;      // [B] or NULL (ones)
    int* cnt;                   // [B][K*C + C*C + C + 1] scratch counters
    double* part;               // [B][gold_blocks(T)] scratch block sums
    int* status;                // status word of the workspace
    float* nll;                 // [B]
    float* grad_em;             // [B][T][C] gradients of the backward pass, corrected in place
    float* grad_trans;          // [C][C]
    float* grad_dur;            // [K][C]
    float* grad_proj_start;     // [B][T][C] or NULL, corrected in place
    float* grad_proj_end;       // [B][T][C] or NULL, corrected in place
};
int gold_blocks(int T);
hipError_t launch_gold(const GoldArgs& g, hipStream_t stream);

// ------------------------------------------------------------------ Viterbi
// chunk length and chunk count of the parallel backtrace
int backtrace_chunk(int T, int C, int K);
int backtrace_chunks(int T, int C, int K);
// the backtrace's chunk tables live in global memory (the chunks' LDS would not hold them)
bool backtrace_global(int T, int C, int K);
// int32 words of that global scratch (0 when the tables fit LDS)
size_t backtrace_scratch_ints(int B, int T, int C, int K);
// vend[b] = {L, c*}: c* the lowest label maximising vfin[b][c] (the values V(L, c) of the
// span that holds L, in its frame); best_score[b] = V(L, c*) + off[b][that span] (NaN for
// an invalid length)
hipError_t launch_vit_final(const double* vfin, const double* off, const int* Leff, int B,
                            int C, int delta, int nspans, int* vend, float* best_score,
                            hipStream_t stream);
// bp: [B][T+1][C]; tr: [B][nch][K*C] and ent: [B][nch] int32 scratch; gscratch: the global
// chunk tables (backtrace_scratch_ints words) or NULL when they fit LDS
hipError_t launch_backtrace(const uint32_t* bp, const int* vend, int B, int T, int C, int K,
                            int32_t* tr, int32_t* ent, int* gscratch, int32_t* labels,
                            uint8_t* seg_start, hipStream_t stream);

}  // namespace semicrf
