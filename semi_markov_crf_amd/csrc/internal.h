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
inline size_t lse_round_lds_bytes(int C, int CP, int P, int CH, bool lin, bool proj) {
    const int cp4 = (CP + 3) / 4 * 4;
    return (size_t)(2 * CH * C + (C + 1) / 2 * 2) * 8 +
           (size_t)((proj ? 10 : 6) * C * CH + (lin ? 2 : 1) * (C + 1) * P + 4 * CP * ROUND +
                    4 * (CP + 1) * ROUND + 2 * cp4 + 16 + 2 * CP * ROUND + 4) * 4 +
           (size_t)2 * CP * 8;
}
// Dynamic LDS of the max-plus round kernel (C <= 16): S chunks [2][C][CH] and S(L) (fp64),
// with projections the chunks' end-side and start-side projections [2][2][C][CH], the
// ring [C+1][P], bulk maxima and their k [2][CP][2][ROUND], rebase shifts [CP rounded to
// 4], a sink and a constant block [12] (fp32).
inline size_t maxplus_round_lds_bytes(int C, int CP, int P, int CH, bool proj) {
    const int cp4 = (CP + 3) / 4 * 4;
    return (size_t)(2 * CH * C + (C + 1) / 2 * 2) * 8 +
           (size_t)((proj ? 4 : 0) * C * CH + (C + 1) * P + 4 * CP * ROUND + cp4 + 12) * 4;
}
// Dynamic LDS of the max-plus sweep: end-side and start-side S chunks [2][2][CH][C]
// (fp64), R ring [C+1][P] and u [2][UP] (fp32).
inline size_t maxplus_lds_bytes(int C, int UP, int P, int CH) {
    return (size_t)(4 * CH * C) * 8 + (size_t)((C + 1) * P + 2 * UP) * 4;
}

enum SweepMode { MODE_FULL = 0, MODE_SPAN = 1 };

struct SweepArgs {
    const double* S;        // [B][T+1][C] centred prefix sums
    const int* Leff;        // [B] clamped length, negated when the input length was invalid
    const float* trans;     // [C][C]
    const float* dur;       // [K][C]
    int B, T, C, K;
    int mode;               // MODE_FULL: grid (B, ndir); MODE_SPAN: grid (nspans, B, ndir)
    int delta;              // checkpoint interval
    int nspans;             // max spans per sequence (ceil(T / delta))
    int write_ckpt;         // FULL mode: write checkpoints at multiples of delta
    int write_xa;           // write per-position X / A (SPAN mode, or FULL with one span)
    // checkpoints [2 dirs][B][nspans][...]; index 0 of the span axis is unused
    float* ck_ring;         // [..][K][C]
    double* ck_base;        // [..][C]
    float* ck_mprev;        // [..][C]
    double* ck_href;        // [..]
    // per-position outputs, natural-log units, [B][T+1][C]
    double* XF;             // forward: alpha[t, c]
    double* AF;             // forward: alpha_bar[t, c] - S[t, c]
    double* XB;             // backward: beta_bar[s, c]
    double* AB;             // backward: beta[u, c] + S[u, c] - S[L, c]
    double* logz;           // [B] forward log Z
    double* logz_b;         // [B] log Z from the backward sweep (consistency check)
    // Viterbi
    uint32_t* bp;           // [2 dirs][B][T+1][C]: (k) | (previous label << 16)
    double* vscore;         // [B] (one-direction sweep)
    int* vcstar;            // [B] final label (one-direction sweep)
    double* vwin;           // [2 dirs][B][K][C] values over the meeting window (round kernel)
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
};

// log-semiring sweep: grid (B, ndir) in MODE_FULL, (nspans, B, ndir) in MODE_SPAN;
// dispatches on cfg.lse.layout to the per-layout translation units
hipError_t launch_lse(const SweepCfg& cfg, const SweepLaunch& a, int ndir, hipStream_t stream);
hipError_t launch_lse_mirror(const SweepCfg& cfg, const SweepLaunch& a, int ndir, hipStream_t stream);
hipError_t launch_lse_plain(const SweepCfg& cfg, const SweepLaunch& a, int ndir, hipStream_t stream);
hipError_t launch_lse_log(const SweepCfg& cfg, const SweepLaunch& a, int ndir, hipStream_t stream);
// round kernels (C <= 16) with boundary projections
hipError_t launch_lse_round_proj(const SweepCfg& cfg, const SweepLaunch& a, int ndir, bool lin,
                                 hipStream_t stream);
hipError_t launch_maxplus_round_proj(const SweepCfg& cfg, const SweepLaunch& a, hipStream_t stream);
// max-plus sweep (Viterbi): MODE_FULL, forward only, grid (B); dispatches on cfg.vit.layout
hipError_t launch_maxplus(const SweepCfg& cfg, const SweepLaunch& a, hipStream_t stream);
hipError_t launch_maxplus_mirror(const SweepCfg& cfg, const SweepLaunch& a, hipStream_t stream);
hipError_t launch_maxplus_plain(const SweepCfg& cfg, const SweepLaunch& a, hipStream_t stream);

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
struct MargArgs {
    const double* S;
    const int* Leff;
    const float* trans;
    const float* dur;
    int B, T, C, K;
    int tile;               // positions per tile
    int kchunk;             // durations per staged chunk
    int ntiles;             // ceil((T+1) / tile)
    const double* XF; const double* AF; const double* XB; const double* AB;
    const double* logz;
    double* Dn;             // [B][T+1][C]: start mass - end mass of segments at each position
    double* dn_tile;        // [B][ntiles][C]: tile sums of Dn
    double* part_dur;       // [B][ntiles][K][C]
    double* part_trans;     // [B][ntiles][C][C]
    float* pstart;          // [B][T][C] or NULL: start mass of segments at each position
    float* pend;            // [B][T][C] or NULL: mass of segments whose last position it is
};
hipError_t launch_marginals(const MargArgs& a, hipStream_t stream);

// mu = prefix sum of Dn, normalised per position; writes marginals, per-tile sums of
// mu and the per-tile mean normaliser.  With pstart / pend (the raw start and end masses
// of k_marginals) also the boundary probability [B][T] and g times the normalised start
// and end marginals [B][T][C] (any of the three outputs may be NULL).
struct BoundaryOut {
    const float* pstart;
    const float* pend;
    const float* grad_log_z;
    float* grad_proj_start;
    float* grad_proj_end;
    float* boundary;
};
hipError_t launch_node_marginals(const double* Dn, const double* dn_off, const int* Leff,
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
                                  int B, int T, int C, int K, int tile, int ntiles,
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
int backtrace_chunk(int C, int K);
int backtrace_chunks(int T, int C, int K);
// split[b] = {t*, c_left, c_right, L}: the best segmentation's boundary in the meeting
// window of the two-direction sweep (bidir), or t* = L and the one-direction sweep's final
// label; best_score[b] its score (NaN for an invalid length)
hipError_t launch_vit_combine(const double* vwin, const float* trans, const int* Leff, int B,
                              int C, int K, bool bidir, const double* vscore, const int* vcstar,
                              int* split, float* best_score, hipStream_t stream);
// bp: [2][B][T+1][C] (part 1: the mirrored sequence); tr: [2][B][nch][K*C] and ent:
// [2][B][nch] int32 scratch
hipError_t launch_backtrace(const uint32_t* bp, const int* split, int B, int T, int C, int K,
                            int32_t* tr, int32_t* ent, int32_t* labels, uint8_t* seg_start,
                            hipStream_t stream);

}  // namespace semicrf
