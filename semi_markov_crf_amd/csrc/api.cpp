// C ABI of the semi-CRF library: argument checks, workspace layout and the launch
// sequence of each call.  See include/semicrf.h for the contract.
#include <math.h>
#include <string.h>

#include <hip/hip_runtime.h>

#include "../../include/semicrf.h"
#include "internal.h"

using namespace semicrf;

namespace {

constexpr size_t ALIGN = 256;
constexpr int MAX_T = 1 << 29;   // keeps position arithmetic (t + delta) inside int

struct Layout {
    int nts = 0, ntm = 0, tm = 0, delta = 0, nspans = 0;
    size_t status = 0, Leff = 0, tsum = 0, toff = 0, ttot = 0, S = 0;
    size_t logz = 0, logzb = 0;
    size_t ckR = 0, ckB = 0, ckM = 0, ckH = 0, XF = 0, AF = 0, XB = 0, AB = 0;
    size_t Dn = 0, dnt = 0, dno = 0, mu = 0, mut = 0, mutot = 0, zt = 0, pd = 0, pt = 0, rps = 0;
    size_t gcnt = 0, gpart = 0, pst = 0, pen = 0;
    size_t bp = 0, vscore = 0, vcstar = 0, vwin = 0, split = 0, btr = 0, bent = 0;
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

bool shape_ok(int B, int T, int C, int K) {
    return B >= 1 && T >= 1 && C >= 1 && K >= 1 && T <= MAX_T && K <= 65535;
}

bool make_layout(int op, int B, int T, int C, int K, int delta, Layout& lo) {
    if (!shape_ok(B, T, C, K)) return false;
    if (!choose_sweep(C, K).ok) return false;
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
    if (op == SEMICRF_OP_LOGZ) {
        lo.logz = m.take(sizeof(double) * B);
    } else if (op == SEMICRF_OP_BACKWARD) {
        lo.delta = resolve_delta(T, K, delta);
        if (lo.delta < 1) return false;
        lo.nspans = (T + lo.delta - 1) / lo.delta;
        lo.tm = marg_tile(C, K);
        lo.ntm = (T + 1 + lo.tm - 1) / lo.tm;
        const size_t nck = (size_t)2 * B * lo.nspans;
        lo.logz = m.take(sizeof(double) * B);
        lo.logzb = m.take(sizeof(double) * B);
        lo.ckR = m.take(sizeof(float) * nck * K * C);
        lo.ckB = m.take(sizeof(double) * nck * C);
        lo.ckM = m.take(sizeof(float) * nck * C);
        lo.ckH = m.take(sizeof(double) * nck);
        lo.XF = m.take(sizeof(double) * BT1C);
        lo.AF = m.take(sizeof(double) * BT1C);
        lo.XB = m.take(sizeof(double) * BT1C);
        lo.AB = m.take(sizeof(double) * BT1C);
        lo.Dn = m.take(sizeof(double) * BT1C);
        lo.dnt = m.take(sizeof(double) * B * lo.ntm * C);
        lo.dno = m.take(sizeof(double) * B * lo.ntm * C);
        lo.mu = m.take(sizeof(float) * B * T * C);
        lo.mut = m.take(sizeof(double) * B * lo.ntm * C);
        lo.mutot = m.take(sizeof(double) * B * C);
        lo.zt = m.take(sizeof(double) * B * lo.ntm);
        lo.pd = m.take(sizeof(double) * B * lo.ntm * K * C);
        lo.pt = m.take(sizeof(double) * B * lo.ntm * C * C);
        lo.rps = m.take(sizeof(double) * reduce_scratch_doubles(C, K));
        // raw start / end masses for the boundary outputs
        lo.pst = m.take(sizeof(float) * (size_t)B * T * C);
        lo.pen = m.take(sizeof(float) * (size_t)B * T * C);
        // gold-segmentation loss (semicrf_nll): counters and block sums
        lo.gcnt = m.take(sizeof(int) * (size_t)B * (K * C + C * C + C + 1));
        lo.gpart = m.take(sizeof(double) * (size_t)B * gold_blocks(T));
    } else if (op == SEMICRF_OP_PREFIX) {
        // S goes to the caller's buffer: drop the internal copy
        lo.total = lo.S;
        return true;
    } else if (op == SEMICRF_OP_VITERBI) {
        lo.bp = m.take(sizeof(uint32_t) * 2 * BT1C);
        lo.vscore = m.take(sizeof(double) * B);
        lo.vcstar = m.take(sizeof(int) * B);
        lo.vwin = m.take(sizeof(double) * 2 * B * K * C);
        lo.split = m.take(sizeof(int) * 4 * B);
        const size_t nch = (size_t)backtrace_chunks(T, C, K);
        lo.btr = m.take(sizeof(int32_t) * 2 * B * nch * K * C);
        lo.bent = m.take(sizeof(int32_t) * 2 * B * nch);
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
    return a;
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
        default: return "unknown status";
    }
}

int semicrf_checkpoint_interval(int T, int K, int delta) { return resolve_delta(T, K, delta); }

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

size_t semicrf_workspace_bytes(int op, int B, int T, int C, int K, int delta) {
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
                    const Proj& pj, int B, int T, int C, int K, hipStream_t stream,
                    void* workspace, size_t workspace_bytes, float* log_z, hipEvent_t* events) {
    int rc = common_checks(em, lengths, trans, dur, B, T, C, K);
    if (rc) return rc;
    if (!log_z) return SEMICRF_ERR_INVALID;
    Layout lo;
    if (!make_layout(SEMICRF_OP_LOGZ, B, T, C, K, 0, lo)) return SEMICRF_ERR_UNSUPPORTED;
    if ((rc = check_ws(workspace, workspace_bytes, lo))) return rc;
    STAGE(0);
    if ((rc = run_prefix(em, lengths, B, T, C, workspace, lo, stream))) return rc;
    STAGE(1);
    const SweepCfg cfg = choose_sweep(C, K);
    SweepLaunch a = base_args(trans, dur, pj, B, T, C, K, workspace, lo);
    a.mode = MODE_FULL;
    a.logz = at<double>(workspace, lo.logz);
    LAUNCH(launch_lse(cfg, a, 1, stream));
    LAUNCH(launch_write_logz(a.logz, B, log_z, stream));
    STAGE(2);
    return SEMICRF_OK;
}

static int run_backward(const float* em, const int32_t* lengths, const float* trans,
                        const float* dur, const Proj& pj, int B, int T, int C, int K, int delta,
                        hipStream_t stream, void* workspace, size_t workspace_bytes,
                        const float* grad_log_z, float* grad_em, float* grad_trans,
                        float* grad_dur, float* marginals, float* log_z, const BoundaryRes& br,
                        hipEvent_t* events) {
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
    a.delta = lo.delta;
    a.nspans = lo.nspans;
    a.ck_ring = at<float>(workspace, lo.ckR);
    a.ck_base = at<double>(workspace, lo.ckB);
    a.ck_mprev = at<float>(workspace, lo.ckM);
    a.ck_href = at<double>(workspace, lo.ckH);
    a.XF = at<double>(workspace, lo.XF);
    a.AF = at<double>(workspace, lo.AF);
    a.XB = at<double>(workspace, lo.XB);
    a.AB = at<double>(workspace, lo.AB);
    a.logz = at<double>(workspace, lo.logz);
    a.logz_b = at<double>(workspace, lo.logzb);
    if (lo.nspans > 1) {
        // streaming sweeps in both directions at once: checkpoints every delta positions
        a.mode = MODE_FULL;
        a.write_ckpt = 1;
        a.write_xa = 0;
        LAUNCH(launch_lse(cfg, a, 2, stream));
    }
    STAGE(2);
    // recompute every checkpoint span in parallel, writing the per-position values
    a.mode = MODE_SPAN;
    a.write_ckpt = 0;
    a.write_xa = 1;
    LAUNCH(launch_lse(cfg, a, 2, stream));
    STAGE(3);

    MargArgs m{};
    m.S = a.S; m.Leff = a.Leff; m.trans = trans; m.dur = dur;
    m.B = B; m.T = T; m.C = C; m.K = K;
    m.tile = lo.tm; m.ntiles = lo.ntm; m.kchunk = marg_kchunk(C, K);
    m.XF = a.XF; m.AF = a.AF; m.XB = a.XB; m.AB = a.AB; m.logz = a.logz;
    m.Dn = at<double>(workspace, lo.Dn);
    m.dn_tile = at<double>(workspace, lo.dnt);
    m.part_dur = at<double>(workspace, lo.pd);
    m.part_trans = at<double>(workspace, lo.pt);
    const bool want_b = br.grad_start || br.grad_end || br.prob;
    if (want_b) {
        m.pstart = at<float>(workspace, lo.pst);
        m.pend = at<float>(workspace, lo.pen);
    }
    LAUNCH(launch_marginals(m, stream));
    STAGE(4);
    LAUNCH(launch_tile_scan(m.dn_tile, B, lo.ntm, C, false, at<double>(workspace, lo.dno), nullptr,
                            stream));
    float* mu = marginals ? marginals : at<float>(workspace, lo.mu);
    BoundaryOut bo{};
    if (want_b) {
        bo.pstart = m.pstart;
        bo.pend = m.pend;
        bo.grad_log_z = grad_log_z;
        bo.grad_proj_start = br.grad_start;
        bo.grad_proj_end = br.grad_end;
        bo.boundary = br.prob;
    }
    LAUNCH(launch_node_marginals(m.Dn, at<double>(workspace, lo.dno), a.Leff, B, T, C, lo.tm,
                                 lo.ntm, mu, at<double>(workspace, lo.mut),
                                 at<double>(workspace, lo.zt), bo, stream));
    LAUNCH(launch_tile_scan(at<double>(workspace, lo.mut), B, lo.ntm, C, false, nullptr,
                            at<double>(workspace, lo.mutot), stream));
    LAUNCH(launch_grad_em(mu, at<double>(workspace, lo.mutot), a.Leff, grad_log_z, B, T, C, grad_em,
                          stream));
    LAUNCH(launch_reduce_partials(m.part_dur, m.part_trans, at<double>(workspace, lo.zt), a.Leff,
                                  grad_log_z, B, T, C, K, lo.tm, lo.ntm,
                                  at<double>(workspace, lo.rps), grad_dur, grad_trans, stream));
    if (log_z) LAUNCH(launch_write_logz(a.logz, B, log_z, stream));
    STAGE(5);
    return SEMICRF_OK;
}

static int run_viterbi(const float* em, const int32_t* lengths, const float* trans,
                       const float* dur, const Proj& pj, int B, int T, int C, int K,
                       hipStream_t stream, void* workspace, size_t workspace_bytes,
                       float* best_score, int32_t* labels, uint8_t* seg_start,
                       hipEvent_t* events) {
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
    a.mode = MODE_FULL;
    a.bp = at<uint32_t>(workspace, lo.bp);
    a.vscore = at<double>(workspace, lo.vscore);
    a.vcstar = at<int>(workspace, lo.vcstar);
    a.vwin = at<double>(workspace, lo.vwin);
    LAUNCH(launch_maxplus(cfg, a, stream));
    STAGE(2);
    int* split = at<int>(workspace, lo.split);
    LAUNCH(launch_vit_combine(a.vwin, trans, a.Leff, B, C, K, cfg.split, a.vscore, a.vcstar,
                              split, best_score, stream));
    LAUNCH(launch_backtrace(a.bp, split, B, T, C, K, at<int32_t>(workspace, lo.btr),
                            at<int32_t>(workspace, lo.bent), labels, seg_start, stream));
    STAGE(3);
    return SEMICRF_OK;
}

int semicrf_logz(const float* em, const int32_t* lengths, const float* trans, const float* dur,
                 const float* proj_start, const float* proj_end, int B, int T, int C, int K,
                 hipStream_t stream, void* workspace, size_t workspace_bytes, float* log_z) {
    return run_logz(em, lengths, trans, dur, Proj{proj_start, proj_end}, B, T, C, K, stream,
                    workspace, workspace_bytes, log_z, nullptr);
}

int semicrf_logz_staged(const float* em, const int32_t* lengths, const float* trans,
                        const float* dur, const float* proj_start, const float* proj_end, int B,
                        int T, int C, int K, hipStream_t stream, void* workspace,
                        size_t workspace_bytes, float* log_z, hipEvent_t* events) {
    if (!events) return SEMICRF_ERR_INVALID;
    return run_logz(em, lengths, trans, dur, Proj{proj_start, proj_end}, B, T, C, K, stream,
                    workspace, workspace_bytes, log_z, events);
}

int semicrf_backward(const float* em, const int32_t* lengths, const float* trans, const float* dur,
                     const float* proj_start, const float* proj_end, int B, int T, int C, int K,
                     int delta, hipStream_t stream, void* workspace, size_t workspace_bytes,
                     const float* grad_log_z, float* grad_em, float* grad_trans, float* grad_dur,
                     float* marginals, float* log_z, float* grad_proj_start,
                     float* grad_proj_end, float* boundary) {
    return run_backward(em, lengths, trans, dur, Proj{proj_start, proj_end}, B, T, C, K, delta,
                        stream, workspace, workspace_bytes, grad_log_z, grad_em, grad_trans,
                        grad_dur, marginals, log_z,
                        BoundaryRes{grad_proj_start, grad_proj_end, boundary}, nullptr);
}

int semicrf_backward_staged(const float* em, const int32_t* lengths, const float* trans,
                            const float* dur, const float* proj_start, const float* proj_end,
                            int B, int T, int C, int K, int delta, hipStream_t stream,
                            void* workspace, size_t workspace_bytes, const float* grad_log_z,
                            float* grad_em, float* grad_trans, float* grad_dur, float* marginals,
                            float* log_z, float* grad_proj_start, float* grad_proj_end,
                            float* boundary, hipEvent_t* events) {
    if (!events) return SEMICRF_ERR_INVALID;
    return run_backward(em, lengths, trans, dur, Proj{proj_start, proj_end}, B, T, C, K, delta,
                        stream, workspace, workspace_bytes, grad_log_z, grad_em, grad_trans,
                        grad_dur, marginals, log_z,
                        BoundaryRes{grad_proj_start, grad_proj_end, boundary}, events);
}

int semicrf_nll(const float* em, const int32_t* lengths, const float* trans, const float* dur,
                const float* proj_start, const float* proj_end, const int32_t* gold_labels,
                const uint8_t* gold_seg_start, int B, int T, int C, int K, int delta,
                hipStream_t stream, void* workspace, size_t workspace_bytes,
                const float* grad_nll, float* nll, float* grad_em, float* grad_trans,
                float* grad_dur, float* grad_proj_start, float* grad_proj_end) {
    if (!gold_labels || !gold_seg_start || !nll) return SEMICRF_ERR_INVALID;
    const Proj pj{proj_start, proj_end};
    int rc = run_backward(em, lengths, trans, dur, pj, B, T, C, K, delta, stream, workspace,
                          workspace_bytes, grad_nll, grad_em, grad_trans, grad_dur, nullptr,
                          nullptr, BoundaryRes{grad_proj_start, grad_proj_end, nullptr}, nullptr);
    if (rc) return rc;
    Layout lo;
    if (!make_layout(SEMICRF_OP_BACKWARD, B, T, C, K, delta, lo)) return SEMICRF_ERR_UNSUPPORTED;
    GoldArgs g{};
    g.S = at<double>(workspace, lo.S);
    g.Leff = at<int>(workspace, lo.Leff);
    g.trans = trans;
    g.dur = dur;
    g.proj_start = proj_start;
    g.proj_end = proj_end;
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
    g.grad_proj_start = grad_proj_start;
    g.grad_proj_end = grad_proj_end;
    LAUNCH(launch_gold(g, stream));
    return SEMICRF_OK;
}

int semicrf_viterbi(const float* em, const int32_t* lengths, const float* trans, const float* dur,
                    const float* proj_start, const float* proj_end, int B, int T, int C, int K,
                    hipStream_t stream, void* workspace, size_t workspace_bytes,
                    float* best_score, int32_t* labels, uint8_t* seg_start) {
    return run_viterbi(em, lengths, trans, dur, Proj{proj_start, proj_end}, B, T, C, K, stream,
                       workspace, workspace_bytes, best_score, labels, seg_start, nullptr);
}

int semicrf_viterbi_staged(const float* em, const int32_t* lengths, const float* trans,
                           const float* dur, const float* proj_start, const float* proj_end,
                           int B, int T, int C, int K, hipStream_t stream, void* workspace,
                           size_t workspace_bytes, float* best_score, int32_t* labels,
                           uint8_t* seg_start, hipEvent_t* events) {
    if (!events) return SEMICRF_ERR_INVALID;
    return run_viterbi(em, lengths, trans, dur, Proj{proj_start, proj_end}, B, T, C, K, stream,
                       workspace, workspace_bytes, best_score, labels, seg_start, events);
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
