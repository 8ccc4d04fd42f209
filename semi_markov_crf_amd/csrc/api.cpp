// C ABI of the semi-CRF library: argument checks, workspace layout and the launch
// sequence of each call.  See include/semicrf.h for the contract.
#include <math.h>
#include <algorithm>
#include <string.h>

#include <mutex>

#include <hip/hip_runtime.h>

#include "../../include/semicrf.h"
#include "internal.h"

using namespace semicrf;

namespace {

constexpr size_t ALIGN = 256;
constexpr int MAX_T = 1 << 29;   // keeps position arithmetic (t + delta) inside int

struct Layout {
    int nts = 0, ntm = 0, tm = 0, tpg = 0, ngm = 0, delta = 0, nspans = 0, ndir = 0, npb = 1;
    size_t status = 0, Leff = 0, tsum = 0, toff = 0, ttot = 0, S = 0;
    size_t logz = 0, logzb = 0;
    size_t head = 0, tail = 0, lzloc = 0, soff = 0, fbad = 0, diag = 0, sstat = 0;
    size_t ckR = 0, ckB = 0, ckM = 0, ckH = 0, XF = 0, XB = 0;
    size_t dnt = 0, dno = 0, mut = 0, mutot = 0, zt = 0, pd = 0, pt = 0, rps = 0, pbp = 0;
    size_t gcnt = 0, gpart = 0;
    size_t bp = 0, vfin = 0, vend = 0, btr = 0, bent = 0, btg = 0;
    size_t xkr = 0;                 // long-duration sweeps: the global ring scratch
    bool has_xkr = false;
    size_t total = 0;
};

struct Bump {
    size_t off = 0;
    size_t take(size_t bytes) {
        const size_t o = off;
        off += (bytes + ALIGN - 1) / ALIGN * ALIGN;
        return o;
    }
};

int resolve_delta(int T, int K, int delta) {
    if (T < 1 || K < 1 || delta < 0) return 0;
    long long d = delta;
    if (d == 0) {
        const long long n = (long long)T * K;
        d = (long long)ceil(sqrt((double)n));
        while (d * d < n) ++d;
        while (d > 1 && (d - 1) * (d - 1) >= n) --d;
    }
    if (d > T) d = T;
    if (d < 1) d = 1;
    return (int)d;
}

// The decode's checkpoint interval outside the round kernels (more than 16 labels, or
// K > 1025).  It starts from ceil(sqrt(T*K)) and halves it when the batch's spans (one
// workgroup each) would leave most compute units idle and a span stays long next to its
// burn-in: with 32 speech-length sequences the halving costs more burn-in than it gains
// (0.53 -> 0.61 ms), so it is not taken there.
int default_delta(int B, int T, int K) {
    const int d = resolve_delta(T, K, 0);
    if (d < 1) return 0;
    const long long spans = (long long)B * ((T + d - 1) / d);
    if (spans <= 128 && d >= 4 * spec_warm(K)) return (d + 1) / 2;
    return d;
}

// Workgroups that one checkpoint span of `op` takes in the span launch: one for log Z;
// for the backward one when the round kernel holds both directions of a span in one
// workgroup (as its launcher decides, without projections), else two.
static int span_workgroups(const SweepCfg& cfg, int op, int C) {
    if (op != SEMICRF_OP_BACKWARD) return 1;
    if (cfg.split && !cfg.xk) {
        const bool lin = (cfg.lse.layout & SWEEP_LINEAR) != 0;
        if (64 + 2 * cfg.NTv <= 512 &&
            2 * lse_round_region_bytes(C, cfg.CPr, cfg.lse.P, cfg.lse.CH, lin, false) <= 150 * 1024)
            return 1;
    }
    return 2;
}

// The default interval of log Z and the backward (delta = 0).  Every span is swept at
// once; a workgroup's sweep takes time in proportion to its span plus its burn-in, and
// once the spans' workgroups outnumber what the compute units run side by side, a CU
// holds two and each takes about twice as long (measured: the sweeps are issue-bound on
// their CU).  So the interval is the one, over every span count n (interval ceil(T/n)),
// that minimises (interval + burn-in) * ceil(workgroups / share), the longer on ties, among
// intervals at least one burn-in long (shorter spans would spend most of their sweep
// burning in, and their seam windows and checkpoints grow with the span count: at
// K = 8000 that kept the backward's workspace at T = 10^6 from doubling).
// share: 224 workgroups (7/8 of the MI355X's 256 CUs, the rest left to a concurrent call
// such as a decode on another stream) for the round kernels, 256 for the others.
// Measured at B = 4, T = 10^5, K = 200 (round kernel, one workgroup per span): a backward
// beside a decode takes 1.74 ms a pair at 1,786 against 1.96 at ceil(sqrt(TK))/2; 32 speech
// sequences (K = 30, C = 39, two workgroups a span) take 0.50 ms at 200 against 0.68 at 155.
int fill_delta(int B, int T, int K, int op, const SweepCfg& cfg, int C) {
    const int d0 = resolve_delta(T, K, 0);
    if (d0 < 1) return 0;
    const long long wps = span_workgroups(cfg, op, C);
    const long long share = (cfg.split && !cfg.xk) ? 256 * 7 / 8 : 256;
    const long long warm = spec_warm(K);
    const long long nmax = std::max<long long>(1, std::min<long long>(T, 8192 / B));
    long long best_d = d0;
    double best = 1e300;
    for (long long n = 1; n <= nmax; ++n) {
        const long long d = (T + n - 1) / n;
        if (n > 1 && d == (T + n - 2) / (n - 1)) continue;   // same interval as n - 1
        if (n > 1 && d < warm) break;   // spans no shorter than their burn-in (and smaller)
        const long long spans = (T + d - 1) / d;
        const long long rounds = (wps * B * spans + share - 1) / share;
        const double f = (double)(d + (spans > 1 ? warm : 0)) * (double)rounds;
        if (f < best || (f == best && d > best_d)) {
            best = f;
            best_d = d;
        }
    }
    return (int)best_d;
}

// The decode's checkpoint interval (it takes none): the span launch's cost model of
// fill_delta where the round kernel runs (one workgroup a span; at B = 4, T = 10^5, K = 200
// beside a backward pass: 1.68 against 1.71 ms a pair with ceil(sqrt(TK))/2, three runs
// each), default_delta otherwise.
int decode_delta(int B, int T, int K, const SweepCfg& cfg, int C) {
    if (cfg.split && !cfg.xk) return fill_delta(B, T, K, SEMICRF_OP_VITERBI, cfg, C);
    return default_delta(B, T, K);
}

bool shape_ok(int B, int T, int C, int K) {
    return B >= 1 && T >= 1 && C >= 1 && K >= 1 && T <= MAX_T && K <= 65535;
}

bool make_layout(int op, int B, int T, int C, int K, int delta, Layout& lo) {
    if (!shape_ok(B, T, C, K)) return false;
    const SweepCfg cfg = choose_sweep(C, K);
    if (!cfg.ok) return false;
    const size_t BT1C = (size_t)B * (T + 1) * C;
    const int TS = scan_tile(C);
    lo.nts = (T + TS - 1) / TS;
    Bump m;
    lo.status = m.take(sizeof(int) * 4);
    lo.Leff = m.take(sizeof(int) * B);
    lo.tsum = m.take(sizeof(double) * B * lo.nts * C);
    lo.toff = m.take(sizeof(double) * B * lo.nts * C);
    lo.ttot = m.take(sizeof(double) * B * C);
    lo.S = m.take(sizeof(double) * BT1C);
    if (op == SEMICRF_OP_LOGZ || op == SEMICRF_OP_BACKWARD || op == SEMICRF_OP_VITERBI) {
        // checkpoint spans: checkpoints, seam windows and frame offsets per direction (the
        // decode runs forward only, with the default interval)
        // delta = 0 (and always for the decode): the batch-aware default interval
        lo.delta = op == SEMICRF_OP_VITERBI ? decode_delta(B, T, K, cfg, C)
                   : delta == 0             ? fill_delta(B, T, K, op, cfg, C)
                                            : resolve_delta(T, K, delta);
        if (lo.delta < 1) return false;
        lo.nspans = (T + lo.delta - 1) / lo.delta;
        lo.ndir = op == SEMICRF_OP_BACKWARD ? 2 : 1;
        const size_t nck = (size_t)lo.ndir * B * lo.nspans;
        lo.logz = m.take(sizeof(double) * B);
        lo.logzb = m.take(sizeof(double) * B);
        lo.ckR = m.take(sizeof(float) * nck * K * C);
        lo.ckB = m.take(sizeof(double) * nck * C);
        lo.ckM = m.take(sizeof(float) * nck * C);
        lo.ckH = m.take(sizeof(double) * nck);
        lo.head = m.take(sizeof(double) * nck * K * C);
        lo.tail = m.take(sizeof(double) * nck * K * C);
        lo.lzloc = m.take(sizeof(double) * lo.ndir * B);
        lo.soff = m.take(sizeof(double) * nck);
        lo.fbad = m.take(sizeof(int) * lo.ndir * B);
        lo.diag = m.take(sizeof(double) * lo.ndir * B * 4);
        lo.sstat = m.take(sizeof(double) * nck * 3);
        if (cfg.xk) {
            // one ring slice per workgroup of the span sweeps (a repair reuses its span's)
            const bool vit = op == SEMICRF_OP_VITERBI;
            const size_t nf = xk_ring_floats(vit ? cfg.xk_vit : cfg.xk_lse, C,
                                             lo.ndir * B * lo.nspans, vit);
            if (nf > 0) {
                lo.xkr = m.take(sizeof(float) * nf);
                lo.has_xkr = true;
            }
        }
    }
    if (op == SEMICRF_OP_LOGZ) {
    } else if (op == SEMICRF_OP_BACKWARD) {
        lo.tm = marg_tile(C, K);
        lo.ntm = (T + 1 + lo.tm - 1) / lo.tm;
        // the messages before the transition step of both directions (k_trans_step turns
        // them into the values after it, in place)
        lo.XF = m.take(sizeof(double) * BT1C);
        lo.XB = m.take(sizeof(double) * BT1C);
        // mu (and before it the in-tile prefix of start - end mass) goes to the caller's
        // marginals or grad_emissions, the raw boundary masses to the boundary outputs
        // themselves
        lo.dnt = m.take(sizeof(double) * B * lo.ntm * C);
        lo.dno = m.take(sizeof(double) * B * lo.ntm * C);
        lo.mut = m.take(sizeof(double) * B * lo.ntm * C);
        lo.mutot = m.take(sizeof(double) * B * C);
        lo.zt = m.take(sizeof(double) * B * lo.ntm);
        lo.tpg = marg_tiles_per_group(B, lo.ntm, C, K);
        lo.ngm = (lo.ntm + lo.tpg - 1) / lo.tpg;
        lo.pd = m.take(sizeof(double) * B * lo.ngm * K * C);
        // label groups' shares of the raw boundary sums (more than one group only)
        lo.npb = (C + marg_labels(C) - 1) / marg_labels(C);
        if (lo.npb > 1) lo.pbp = m.take(sizeof(float) * (size_t)lo.npb * B * T);
        lo.pt = m.take(sizeof(double) * B * lo.ngm * C * C);
        lo.rps = m.take(sizeof(double) * reduce_scratch_doubles(C, K));
        // gold-segmentation loss (semicrf_nll): counters and block sums
        lo.gcnt = m.take(sizeof(int) * (size_t)B * (K * C + C * C + C + 1));
        lo.gpart = m.take(sizeof(double) * (size_t)B * gold_blocks(T));
    } else if (op == SEMICRF_OP_PREFIX) {
        // S goes to the caller's buffer: drop the internal copy
        lo.total = lo.S;
        return true;
    } else if (op == SEMICRF_OP_VITERBI) {
        lo.bp = m.take(sizeof(uint32_t) * BT1C);
        lo.vfin = m.take(sizeof(double) * B * C);
        lo.vend = m.take(sizeof(int) * 2 * B);
        const size_t nch = (size_t)backtrace_chunks(T, C, K);
        lo.btr = m.take(sizeof(int32_t) * B * nch * K * C);
        lo.bent = m.take(sizeof(int32_t) * B * nch);
        lo.btg = m.take(sizeof(int32_t) * backtrace_scratch_ints(B, T, C, K));
    } else {
        return false;
    }
    lo.total = m.off;
    return true;
}

template <class P>
P* at(void* ws, size_t off) {
    return reinterpret_cast<P*>(static_cast<char*>(ws) + off);
}

int check_ws(void* ws, size_t have, const Layout& lo) {
    if (!ws || have < lo.total || (reinterpret_cast<uintptr_t>(ws) % ALIGN) != 0)
        return SEMICRF_ERR_WORKSPACE;
    return SEMICRF_OK;
}

#define LAUNCH(expr)                                   \
    do {                                               \
        if ((expr) != hipSuccess) return SEMICRF_ERR_DEVICE; \
    } while (0)

// Optional stage timing: events[i] is recorded on the stream before stage i.
#define STAGE(i)                                                                   \
    do {                                                                           \
        if (events && hipEventRecord(events[i], stream) != hipSuccess)             \
            return SEMICRF_ERR_DEVICE;                                             \
    } while (0)

// centring + prefix sums: fills Leff, status and S
int run_prefix(const float* em, const int32_t* lengths, int B, int T, int C, void* ws,
               const Layout& lo, hipStream_t st) {
    int* Leff = at<int>(ws, lo.Leff);
    LAUNCH(launch_em_tile_sums(em, lengths, B, T, C, at<double>(ws, lo.tsum), Leff, st));
    LAUNCH(launch_tile_scan(at<double>(ws, lo.tsum), B, lo.nts, C, false, at<double>(ws, lo.toff),
                            at<double>(ws, lo.ttot), st));
    LAUNCH(launch_prefix(em, Leff, B, T, C, at<double>(ws, lo.toff), at<double>(ws, lo.ttot),
                         at<double>(ws, lo.S), at<int>(ws, lo.status), st));
    return SEMICRF_OK;
}

// optional boundary projections (inputs) and boundary outputs of the backward pass
struct Proj {
    const float* start;
    const float* end;
};
struct BoundaryRes {
    float* grad_start;
    float* grad_end;
    float* prob;
    float* node_mass;
};

// speculative spans: tolerance of the seam check and its optional reports
struct SpecOpt {
    double tol;
    float* bound;
    int* repairs;
};

SweepLaunch base_args(const float* trans, const float* dur, const Proj& pj, int B, int T, int C,
                      int K, void* ws, const Layout& lo) {
    SweepLaunch a{};
    a.S = at<double>(ws, lo.S);
    a.proj_start = pj.start;
    a.proj_end = pj.end;
    a.Leff = at<int>(ws, lo.Leff);
    a.trans = trans;
    a.dur = dur;
    a.B = B; a.T = T; a.C = C; a.K = K;
    a.delta = T;
    a.nspans = 1;
    if (lo.ndir > 0) {
        a.delta = lo.delta;
        a.nspans = lo.nspans;
        a.warm = spec_warm(K);
        a.logz = at<double>(ws, lo.logz);
        a.logz_b = at<double>(ws, lo.logzb);
        a.ck_ring = at<float>(ws, lo.ckR);
        a.ck_base = at<double>(ws, lo.ckB);
        a.ck_mprev = at<float>(ws, lo.ckM);
        a.ck_href = at<double>(ws, lo.ckH);
        a.head = at<double>(ws, lo.head);
        a.tail = at<double>(ws, lo.tail);
        a.lzloc = at<double>(ws, lo.lzloc);
        a.first_bad = at<int>(ws, lo.fbad);
        a.off = at<double>(ws, lo.soff);
        if (lo.has_xkr) a.xk_ring = at<float>(ws, lo.xkr);
    }
    return a;
}

// Every checkpoint span swept at once (MODE_SPEC), the seam check, and the sequential
// repair from the first failed seam (MODE_REPAIR; its workgroups exit at once where no seam
// failed).  Leaves log Z in a.logz (and a.logz_b with two directions) and, with write_xa,
// the per-position outputs in their spans' frames with the offsets in a.off.
int run_spans(const SweepCfg& cfg, SweepLaunch a, int ndir, const Layout& lo, void* ws,
              const SpecOpt& so, hipStream_t stream, hipEvent_t* events, int stage) {
    a.mode = MODE_SPEC;
    LAUNCH(launch_lse(cfg, a, ndir, stream));
    if (events && stage >= 0 && hipEventRecord(events[stage], stream) != hipSuccess)
        return SEMICRF_ERR_DEVICE;
    SeamArgs sa{};
    sa.head = a.head;
    sa.tail = a.tail;
    sa.lzloc = a.lzloc;
    sa.Leff = a.Leff;
    sa.B = a.B; sa.C = a.C; sa.K = a.K; sa.delta = a.delta; sa.nspans = a.nspans;
    sa.tol = so.tol;
    sa.off = at<double>(ws, lo.soff);
    sa.first_bad = at<int>(ws, lo.fbad);
    sa.logz = a.logz;
    sa.logz_b = a.logz_b;
    sa.diag = at<double>(ws, lo.diag);
    sa.stats = at<double>(ws, lo.sstat);
    LAUNCH(launch_seam(sa, ndir, stream));
    a.mode = MODE_REPAIR;
    LAUNCH(launch_lse(cfg, a, ndir, stream));
    LAUNCH(launch_seam_report(sa.diag, a.B, ndir, so.bound, so.repairs, stream));
    return SEMICRF_OK;
}

}  // namespace

extern "C" {

const char* semicrf_status_string(int status) {
    switch (status) {
        case SEMICRF_OK: return "ok";
        case SEMICRF_ERR_INVALID: return "invalid argument";
        case SEMICRF_ERR_WORKSPACE: return "workspace missing, too small or misaligned";
        case SEMICRF_ERR_UNSUPPORTED: return "unsupported shape";
        case SEMICRF_ERR_DEVICE: return "device error";
        case SEMICRF_ERR_UNIMPLEMENTED: return "not implemented";
        default: return "unknown status";
    }
}

int semicrf_checkpoint_interval(int T, int K, int delta) { return resolve_delta(T, K, delta); }

int semicrf_default_interval(semicrf_op op, int B, int T, int C, int K) {
    if (!shape_ok(B, T, C, K)) return 0;
    if (op != SEMICRF_OP_LOGZ && op != SEMICRF_OP_BACKWARD && op != SEMICRF_OP_VITERBI) return 0;
    const SweepCfg cfg = choose_sweep(C, K);
    if (!cfg.ok) return 0;
    if (op == SEMICRF_OP_VITERBI) return decode_delta(B, T, K, cfg, C);
    return fill_delta(B, T, K, op, cfg, C);
}

int semicrf_prefix(const float* em, const int32_t* lengths, int B, int T, int C,
                   hipStream_t stream, void* workspace, size_t workspace_bytes, double* S) {
    if (!em || !lengths || !S) return SEMICRF_ERR_INVALID;
    if (!shape_ok(B, T, C, 1)) return SEMICRF_ERR_INVALID;
    Layout lo;
    if (!make_layout(SEMICRF_OP_PREFIX, B, T, C, 1, 0, lo)) return SEMICRF_ERR_UNSUPPORTED;
    int rc = check_ws(workspace, workspace_bytes, lo);
    if (rc) return rc;
    int* Leff = at<int>(workspace, lo.Leff);
    LAUNCH(launch_em_tile_sums(em, lengths, B, T, C, at<double>(workspace, lo.tsum), Leff, stream));
    LAUNCH(launch_tile_scan(at<double>(workspace, lo.tsum), B, lo.nts, C, false,
                            at<double>(workspace, lo.toff), at<double>(workspace, lo.ttot), stream));
    LAUNCH(launch_prefix(em, Leff, B, T, C, at<double>(workspace, lo.toff),
                         at<double>(workspace, lo.ttot), S, at<int>(workspace, lo.status), stream));
    return SEMICRF_OK;
}

size_t semicrf_workspace_bytes(semicrf_op op, int B, int T, int C, int K, int delta) {
    Layout lo;
    if (!make_layout(op, B, T, C, K, delta, lo)) return 0;
    return lo.total;
}

static int common_checks(const float* em, const int32_t* lengths, const float* trans,
                         const float* dur, int B, int T, int C, int K) {
    if (!em || !lengths || !trans || !dur) return SEMICRF_ERR_INVALID;
    if (!shape_ok(B, T, C, K)) return SEMICRF_ERR_INVALID;
    if (!choose_sweep(C, K).ok) return SEMICRF_ERR_UNSUPPORTED;
    return SEMICRF_OK;
}

static int run_logz(const float* em, const int32_t* lengths, const float* trans, const float* dur,
                    const Proj& pj, int B, int T, int C, int K, int delta, hipStream_t stream,
                    void* workspace, size_t workspace_bytes, float* log_z, const SpecOpt& so,
                    hipEvent_t* events) {
    int rc = common_checks(em, lengths, trans, dur, B, T, C, K);
    if (rc) return rc;
    if (!log_z || delta < 0) return SEMICRF_ERR_INVALID;
    Layout lo;
    if (!make_layout(SEMICRF_OP_LOGZ, B, T, C, K, delta, lo)) return SEMICRF_ERR_UNSUPPORTED;
    if ((rc = check_ws(workspace, workspace_bytes, lo))) return rc;
    STAGE(0);
    if ((rc = run_prefix(em, lengths, B, T, C, workspace, lo, stream))) return rc;
    STAGE(1);
    const SweepCfg cfg = choose_sweep(C, K);
    SweepLaunch a = base_args(trans, dur, pj, B, T, C, K, workspace, lo);
    // every checkpoint span at once, then the seam check
    a.write_xa = 0;
    if ((rc = run_spans(cfg, a, 1, lo, workspace, so, stream, nullptr, -1))) return rc;
    LAUNCH(launch_write_logz(a.logz, B, log_z, stream));
    STAGE(2);
    return SEMICRF_OK;
}

static int run_backward(const float* em, const int32_t* lengths, const float* trans,
                        const float* dur, const Proj& pj, int B, int T, int C, int K, int delta,
                        hipStream_t stream, void* workspace, size_t workspace_bytes,
                        const float* grad_log_z, float* grad_em, float* grad_trans,
                        float* grad_dur, float* marginals, float* log_z, const BoundaryRes& br,
                        const SpecOpt& so, hipEvent_t* events) {
    int rc = common_checks(em, lengths, trans, dur, B, T, C, K);
    if (rc) return rc;
    if (!grad_em || !grad_trans || !grad_dur || delta < 0) return SEMICRF_ERR_INVALID;
    Layout lo;
    if (!make_layout(SEMICRF_OP_BACKWARD, B, T, C, K, delta, lo)) return SEMICRF_ERR_UNSUPPORTED;
    if ((rc = check_ws(workspace, workspace_bytes, lo))) return rc;
    STAGE(0);
    if ((rc = run_prefix(em, lengths, B, T, C, workspace, lo, stream))) return rc;
    STAGE(1);
    const SweepCfg cfg = choose_sweep(C, K);
    SweepLaunch a = base_args(trans, dur, pj, B, T, C, K, workspace, lo);
    a.XF = at<double>(workspace, lo.XF);
    a.XB = at<double>(workspace, lo.XB);
    a.write_xa = 1;
    // every checkpoint span of both directions at once with its per-position values, then
    // the seam check and the repair of failed seams
    if ((rc = run_spans(cfg, a, 2, lo, workspace, so, stream, events, 2))) return rc;
    STAGE(3);

    TransStepArgs ts{};
    ts.S = a.S; ts.Leff = a.Leff; ts.trans = trans;
    ts.B = B; ts.T = T; ts.C = C;
    ts.tile = lo.tm; ts.ntiles = lo.ntm; ts.tpg = lo.tpg; ts.ngroups = lo.ngm;
    ts.XF = a.XF; ts.XB = a.XB;
    ts.proj_start = pj.start; ts.proj_end = pj.end;
    ts.logz = a.logz;
    ts.off = a.off; ts.delta = lo.delta; ts.nspans = lo.nspans;
    ts.part_trans = at<double>(workspace, lo.pt);
    LAUNCH(launch_trans_step(ts, stream));

    MargArgs m{};
    m.S = a.S; m.Leff = a.Leff; m.dur = dur;
    m.B = B; m.T = T; m.C = C; m.K = K;
    m.tile = lo.tm; m.ntiles = lo.ntm; m.kchunk = marg_kchunk(C, K);
    m.tpg = lo.tpg; m.ngroups = lo.ngm;
    m.AF = a.XF; m.AB = a.XB;
    m.dn_tile = at<double>(workspace, lo.dnt);
    m.part_dur = at<double>(workspace, lo.pd);
    // raw boundary masses straight into the outputs that k_node_marginals rescales in place
    m.pstart = br.grad_start;
    m.pend = br.grad_end;
    m.pbsum = br.prob;
    m.cg = marg_labels(C);
    m.pb_part = lo.npb > 1 ? at<float>(workspace, lo.pbp) : nullptr;
    // mu lives in the caller's marginals, else in grad_emissions (k_grad_em then works in
    // place); k_marginals leaves the in-tile prefix there first
    float* mu = marginals ? marginals : grad_em;
    m.Dloc = mu;
    LAUNCH(launch_marginals(m, stream));
    STAGE(4);
    LAUNCH(launch_tile_scan(m.dn_tile, B, lo.ntm, C, false, at<double>(workspace, lo.dno), nullptr,
                            stream));
    BoundaryOut bo{};
    bo.grad_log_z = grad_log_z;
    bo.grad_proj_start = br.grad_start;
    bo.grad_proj_end = br.grad_end;
    bo.boundary = br.prob;
    bo.node_mass = br.node_mass;
    bo.pb_part = (lo.npb > 1 && br.prob) ? m.pb_part : nullptr;
    bo.npb = lo.npb;
    LAUNCH(launch_node_marginals(m.Dloc, at<double>(workspace, lo.dno), a.Leff, B, T, C, lo.tm,
                                 lo.ntm, mu, at<double>(workspace, lo.mut),
                                 at<double>(workspace, lo.zt), bo, stream));
    LAUNCH(launch_tile_scan(at<double>(workspace, lo.mut), B, lo.ntm, C, false, nullptr,
                            at<double>(workspace, lo.mutot), stream));
    LAUNCH(launch_grad_em(mu, at<double>(workspace, lo.mutot), a.Leff, grad_log_z, B, T, C, grad_em,
                          stream));
    LAUNCH(launch_reduce_partials(m.part_dur, ts.part_trans, at<double>(workspace, lo.zt), a.Leff,
                                  grad_log_z, B, C, K, lo.tm, lo.ntm, lo.tpg,
                                  at<double>(workspace, lo.rps), grad_dur, grad_trans, stream));
    if (log_z) LAUNCH(launch_write_logz(a.logz, B, log_z, stream));
    STAGE(5);
    return SEMICRF_OK;
}

static int run_viterbi(const float* em, const int32_t* lengths, const float* trans,
                       const float* dur, const Proj& pj, int B, int T, int C, int K,
                       hipStream_t stream, void* workspace, size_t workspace_bytes,
                       float* best_score, int32_t* labels, uint8_t* seg_start,
                       const SpecOpt& so, hipEvent_t* events) {
    int rc = common_checks(em, lengths, trans, dur, B, T, C, K);
    if (rc) return rc;
    if (!best_score || !labels || !seg_start) return SEMICRF_ERR_INVALID;
    Layout lo;
    if (!make_layout(SEMICRF_OP_VITERBI, B, T, C, K, 0, lo)) return SEMICRF_ERR_UNSUPPORTED;
    if ((rc = check_ws(workspace, workspace_bytes, lo))) return rc;
    STAGE(0);
    if ((rc = run_prefix(em, lengths, B, T, C, workspace, lo, stream))) return rc;
    STAGE(1);
    const SweepCfg cfg = choose_sweep(C, K);
    SweepLaunch a = base_args(trans, dur, pj, B, T, C, K, workspace, lo);
    a.bp = at<uint32_t>(workspace, lo.bp);
    a.vfin = at<double>(workspace, lo.vfin);
    // every checkpoint span of the forward decode at once, the seam check (the frame
    // offsets, no log Z), the in-order repair from a failed seam, the final label
    a.mode = MODE_SPEC;
    LAUNCH(launch_maxplus(cfg, a, stream));
    SeamArgs sa{};
    sa.head = a.head;
    sa.tail = a.tail;
    sa.lzloc = a.lzloc;
    sa.Leff = a.Leff;
    sa.B = B; sa.C = C; sa.K = K; sa.delta = a.delta; sa.nspans = a.nspans;
    sa.tol = so.tol;
    sa.off = at<double>(workspace, lo.soff);
    sa.first_bad = at<int>(workspace, lo.fbad);
    sa.logz = a.logz;
    sa.logz_b = a.logz_b;
    sa.diag = at<double>(workspace, lo.diag);
    sa.stats = at<double>(workspace, lo.sstat);
    LAUNCH(launch_seam(sa, 1, stream));
    a.mode = MODE_REPAIR;
    LAUNCH(launch_maxplus(cfg, a, stream));
    int* vend = at<int>(workspace, lo.vend);
    LAUNCH(launch_vit_final(a.vfin, sa.off, a.Leff, B, C, a.delta, a.nspans, vend, best_score,
                            stream));
    LAUNCH(launch_seam_report(sa.diag, B, 1, so.bound, so.repairs, stream));
    STAGE(2);
    LAUNCH(launch_backtrace(a.bp, vend, B, T, C, K, at<int32_t>(workspace, lo.btr),
                            at<int32_t>(workspace, lo.bent),
                            backtrace_global(T, C, K) ? at<int>(workspace, lo.btg) : nullptr, labels,
                            seg_start, stream));
    STAGE(3);
    return SEMICRF_OK;
}

namespace {

const semicrf_options kNoOptions{};

const semicrf_options& opts(const semicrf_options* o) { return o ? *o : kNoOptions; }

SpecOpt spec_opt(const semicrf_options& o) {
    return SpecOpt{o.seam_tolerance == 0.0 ? SEAM_TOL : o.seam_tolerance, o.seam_bound,
                   o.seam_repairs};
}

}  // namespace

int semicrf_logz(const float* em, const int32_t* lengths, const float* trans, const float* dur,
                 int B, int T, int C, int K, int delta, hipStream_t stream, void* workspace,
                 size_t workspace_bytes, float* log_z) {
    return semicrf_logz_ex(em, lengths, trans, dur, B, T, C, K, delta, stream, workspace,
                           workspace_bytes, log_z, nullptr);
}

int semicrf_logz_ex(const float* em, const int32_t* lengths, const float* trans,
                    const float* dur, int B, int T, int C, int K, int delta, hipStream_t stream,
                    void* workspace, size_t workspace_bytes, float* log_z,
                    const semicrf_options* options) {
    const semicrf_options& o = opts(options);
    if (delta < 0) return SEMICRF_ERR_INVALID;
    return run_logz(em, lengths, trans, dur, Proj{o.proj_start, o.proj_end}, B, T, C, K, delta,
                    stream, workspace, workspace_bytes, log_z, spec_opt(o), o.events);
}

int semicrf_backward(const float* em, const int32_t* lengths, const float* trans, const float* dur,
                     int B, int T, int C, int K, int delta, hipStream_t stream, void* workspace,
                     size_t workspace_bytes, const float* grad_log_z, float* grad_em,
                     float* grad_trans, float* grad_dur, float* marginals, float* log_z) {
    return semicrf_backward_ex(em, lengths, trans, dur, B, T, C, K, delta, stream, workspace,
                               workspace_bytes, grad_log_z, grad_em, grad_trans, grad_dur,
                               marginals, log_z, nullptr);
}

int semicrf_backward_ex(const float* em, const int32_t* lengths, const float* trans,
                        const float* dur, int B, int T, int C, int K, int delta,
                        hipStream_t stream, void* workspace, size_t workspace_bytes,
                        const float* grad_log_z, float* grad_em, float* grad_trans,
                        float* grad_dur, float* marginals, float* log_z,
                        const semicrf_options* options) {
    const semicrf_options& o = opts(options);
    return run_backward(em, lengths, trans, dur, Proj{o.proj_start, o.proj_end}, B, T, C, K,
                        delta, stream, workspace, workspace_bytes, grad_log_z, grad_em,
                        grad_trans, grad_dur, marginals, log_z,
                        BoundaryRes{o.grad_proj_start, o.grad_proj_end, o.boundary, o.node_mass},
                        spec_opt(o), o.events);
}

int semicrf_nll(const float* em, const int32_t* lengths, const float* trans, const float* dur,
                const int32_t* gold_labels, const uint8_t* gold_seg_start, int B, int T, int C,
                int K, int delta, hipStream_t stream, void* workspace, size_t workspace_bytes,
                const float* grad_nll, float* nll, float* grad_em, float* grad_trans,
                float* grad_dur, const semicrf_options* options) {
    const semicrf_options& o = opts(options);
    if (!gold_labels || !gold_seg_start || !nll) return SEMICRF_ERR_INVALID;
    if (o.boundary || o.node_mass || o.events) return SEMICRF_ERR_INVALID;
    const Proj pj{o.proj_start, o.proj_end};
    int rc = run_backward(em, lengths, trans, dur, pj, B, T, C, K, delta, stream, workspace,
                          workspace_bytes, grad_nll, grad_em, grad_trans, grad_dur, nullptr,
                          nullptr, BoundaryRes{o.grad_proj_start, o.grad_proj_end, nullptr, nullptr},
                          spec_opt(o), nullptr);
    if (rc) return rc;
    Layout lo;
    if (!make_layout(SEMICRF_OP_BACKWARD, B, T, C, K, delta, lo)) return SEMICRF_ERR_UNSUPPORTED;
    GoldArgs g{};
    g.S = at<double>(workspace, lo.S);
    g.Leff = at<int>(workspace, lo.Leff);
    g.trans = trans;
    g.dur = dur;
    g.proj_start = o.proj_start;
    g.proj_end = o.proj_end;
    g.labels = gold_labels;
    g.seg_start = gold_seg_start;
    g.B = B; g.T = T; g.C = C; g.K = K;
    g.logz = at<double>(workspace, lo.logz);
    g.grad_nll = grad_nll;
    g.cnt = at<int>(workspace, lo.gcnt);
    g.part = at<double>(workspace, lo.gpart);
    g.status = at<int>(workspace, lo.status);
    g.nll = nll;
    g.grad_em = grad_em;
    g.grad_trans = grad_trans;
    g.grad_dur = grad_dur;
    g.grad_proj_start = o.grad_proj_start;
    g.grad_proj_end = o.grad_proj_end;
    LAUNCH(launch_gold(g, stream));
    return SEMICRF_OK;
}

int semicrf_viterbi(const float* em, const int32_t* lengths, const float* trans, const float* dur,
                    int B, int T, int C, int K, hipStream_t stream, void* workspace,
                    size_t workspace_bytes, float* best_score, int32_t* labels,
                    uint8_t* seg_start) {
    return semicrf_viterbi_ex(em, lengths, trans, dur, B, T, C, K, stream, workspace,
                              workspace_bytes, best_score, labels, seg_start, nullptr);
}

int semicrf_viterbi_ex(const float* em, const int32_t* lengths, const float* trans,
                       const float* dur, int B, int T, int C, int K, hipStream_t stream,
                       void* workspace, size_t workspace_bytes, float* best_score,
                       int32_t* labels, uint8_t* seg_start, const semicrf_options* options) {
    const semicrf_options& o = opts(options);
    if (o.grad_proj_start || o.grad_proj_end || o.boundary || o.node_mass)
        return SEMICRF_ERR_INVALID;
    return run_viterbi(em, lengths, trans, dur, Proj{o.proj_start, o.proj_end}, B, T, C, K,
                       stream, workspace, workspace_bytes, best_score, labels, seg_start,
                       spec_opt(o), o.events);
}

}  // extern "C"

// ---------------------------------------------------------------- no-allocation variant
namespace {

// The workspace of semicrf_logz_static: one copy per GPU, in the code object's device
// memory.  Host code never passes `scratch` itself (on the host it only names a
// stand-in): it passes the device address hipGetSymbolAddress returns for each device.
static __device__ __align__(256) unsigned char scratch[SEMICRF_STATIC_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

// Device address of `scratch` on the device of `stream`, looked up once per device with
// that device current.
int static_scratch(hipStream_t stream, void** out) {
    int cur = 0;
    if (hipGetDevice(&cur) != hipSuccess) return SEMICRF_ERR_DEVICE;
    int dev = cur;
    if (stream && hipStreamGetDevice(stream, &dev) != hipSuccess) return SEMICRF_ERR_DEVICE;
    if (dev < 0 || dev >= kMaxDevices) return SEMICRF_ERR_DEVICE;
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (!g_scratch_ptr[dev]) {
        if (dev != cur && hipSetDevice(dev) != hipSuccess) return SEMICRF_ERR_DEVICE;
        void* ptr = nullptr;
        const hipError_t e = hipGetSymbolAddress((void**)&ptr, HIP_SYMBOL(scratch));
        if (dev != cur && hipSetDevice(cur) != hipSuccess) return SEMICRF_ERR_DEVICE;
        if (e != hipSuccess || !ptr) return SEMICRF_ERR_DEVICE;
        g_scratch_ptr[dev] = ptr;
    }
    *out = g_scratch_ptr[dev];
    return SEMICRF_OK;
}

}  // namespace

extern "C" {

int semicrf_logz_static(const float* em, const int32_t* lengths, const float* trans,
                        const float* dur, int B, int T, int C, int K, int delta,
                        hipStream_t stream, float* log_z) {
    int rc = common_checks(em, lengths, trans, dur, B, T, C, K);
    if (rc) return rc;
    if (!log_z || delta < 0) return SEMICRF_ERR_INVALID;
    Layout lo;
    if (!make_layout(SEMICRF_OP_LOGZ, B, T, C, K, delta, lo)) return SEMICRF_ERR_UNSUPPORTED;
    if (lo.total > SEMICRF_STATIC_SCRATCH_BYTES) return SEMICRF_ERR_WORKSPACE;
    void* ws = nullptr;
    if ((rc = static_scratch(stream, &ws))) return rc;
    return run_logz(em, lengths, trans, dur, Proj{nullptr, nullptr}, B, T, C, K, delta, stream,
                    ws, SEMICRF_STATIC_SCRATCH_BYTES, log_z, SpecOpt{SEAM_TOL, nullptr, nullptr},
                    nullptr);
}

int semicrf_read_status(const void* workspace, hipStream_t stream) {
    if (!workspace) return SEMICRF_ERR_WORKSPACE;
    if (hipStreamSynchronize(stream) != hipSuccess) return SEMICRF_ERR_DEVICE;
    int flag = 0;
    if (hipMemcpy(&flag, workspace, sizeof(int), hipMemcpyDeviceToHost) != hipSuccess)
        return SEMICRF_ERR_DEVICE;
    return flag ? SEMICRF_ERR_INVALID : SEMICRF_OK;
}

}  // extern "C"
