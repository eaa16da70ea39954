// fwpkm_api.cpp -- the C ABI of include/fwpkm.h: argument validation,
// workspace carving and the kernel sequence of each entry point.
//
// Per chunk of the causal loop ("Fast-weight Product Key Memory",
// paperlayer.ai 3 and 3.1: read a chunk with the state left by the previous
// one, then write):
//   sweep(select|stats)  scores, top-k, weights, usage partial sums
//   gather               v_hat, o, residual r
//   sort passes          reads ordered by slot
//   scatter + fixup      read-count-normalised V write
//   pbar                 log pbar
//   sweep(rowstat)       Z_t, m_t
//   kgrad                K1/K2 step and their new norms
#include "../../include/fwpkm.h"
#include "fwpkm_internal.h"

#include <algorithm>
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <mutex>
#include <string>
#include <vector>

using namespace fwpkm;

namespace {

thread_local std::string g_err;

int fail(int code, const char* fmt, ...) {
    char buf[512];
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(buf, sizeof buf, fmt, ap);
    va_end(ap);
    g_err = buf;
    return code;
}

int ok() {
    g_err.clear();
    return FWPKM_OK;
}

// ---------------------------------------------------------------------------
// opt-in kernel timing: HIP events around each kernel family launch
// ---------------------------------------------------------------------------
struct TimedPair {
    int family;
    hipEvent_t start, stop;
};

struct Timing {
    std::mutex mu;
    bool on = false;
    std::vector<hipEvent_t> pool;
    std::vector<TimedPair> pending;
    double ms[FWPKM_K_COUNT] = {};
    int64_t launches[FWPKM_K_COUNT] = {};

    hipEvent_t get() {
        if (!pool.empty()) {
            hipEvent_t e = pool.back();
            pool.pop_back();
            return e;
        }
        hipEvent_t e = nullptr;
        if (hipEventCreate(&e) != hipSuccess) return nullptr;
        return e;
    }
};

Timing& timing() {
    static Timing t;
    return t;
}

// Brackets one kernel family launch with events when timing is on.
class TimedLaunch {
  public:
    TimedLaunch(int family, hipStream_t s) : family_(family), s_(s) {
        Timing& t = timing();
        if (!t.on) return;
        std::lock_guard<std::mutex> lk(t.mu);
        start_ = t.get();
        stop_ = t.get();
        if (!start_ || !stop_ || hipEventRecord(start_, s_) != hipSuccess) drop(t);
    }
    ~TimedLaunch() {
        if (!start_ || !stop_) return;
        Timing& t = timing();
        std::lock_guard<std::mutex> lk(t.mu);
        if (hipEventRecord(stop_, s_) != hipSuccess) {
            drop(t);
            return;
        }
        t.pending.push_back({family_, start_, stop_});
    }

  private:
    void drop(Timing& t) {
        if (start_) t.pool.push_back(start_);
        if (stop_) t.pool.push_back(stop_);
        start_ = stop_ = nullptr;
    }
    int family_;
    hipStream_t s_;
    hipEvent_t start_ = nullptr, stop_ = nullptr;
};

// The value stream and the selection stream of fwpkm_forward_seq with their
// fork/join events, one set per (host thread, device of the caller's
// stream), created on the first multi-stream call and kept until
// fwpkm_release_streams() on that thread (or the end of the process).
struct Aux {
    hipStream_t sv = nullptr, sx = nullptr;
    hipEvent_t ev_start = nullptr, ev_sel = nullptr, ev_end = nullptr, ev_scored = nullptr, ev_sorted = nullptr;
    hipEvent_t ev_write[2] = {nullptr, nullptr};
};

thread_local std::vector<Aux*> t_aux;  // indexed by device

// Destroys one set (its streams first wait for their work).
hipError_t aux_destroy(Aux* a) {
    hipError_t first = hipSuccess;
    auto keep = [&](hipError_t e) {
        if (first == hipSuccess) first = e;
    };
    for (hipStream_t st : {a->sv, a->sx})
        if (st) {
            keep(hipStreamSynchronize(st));
            keep(hipStreamDestroy(st));
        }
    for (hipEvent_t ev : {a->ev_start, a->ev_sel, a->ev_end, a->ev_scored, a->ev_sorted, a->ev_write[0],
                          a->ev_write[1]})
        if (ev) keep(hipEventDestroy(ev));
    delete a;
    return first;
}

// Device that work enqueued on `s` runs on (the current device for the
// null stream).
hipError_t stream_device(hipStream_t s, int* dev) {
    if (!s) return hipGetDevice(dev);
    return hipStreamGetDevice(s, dev);
}

hipError_t aux_streams(hipStream_t caller, Aux** out) {
    int dev = 0;
    hipError_t e = stream_device(caller, &dev);
    if (e != hipSuccess) return e;
    if (dev < 0) return hipErrorInvalidDevice;
    if (static_cast<int>(t_aux.size()) <= dev) t_aux.resize(dev + 1, nullptr);
    if (!t_aux[dev]) {
        // create them on the caller's device, then restore the current one
        int cur = 0;
        if ((e = hipGetDevice(&cur)) != hipSuccess) return e;
        if (cur != dev && (e = hipSetDevice(dev)) != hipSuccess) return e;
        Aux* a = new Aux();
        e = hipStreamCreateWithFlags(&a->sv, hipStreamNonBlocking);
        if (e == hipSuccess) e = hipStreamCreateWithFlags(&a->sx, hipStreamNonBlocking);
        hipEvent_t* evs[7] = {&a->ev_start, &a->ev_sel,      &a->ev_end,     &a->ev_scored,
                              &a->ev_sorted, &a->ev_write[0], &a->ev_write[1]};
        for (hipEvent_t* ev : evs)
            if (e == hipSuccess) e = hipEventCreateWithFlags(ev, hipEventDisableTiming);
        if (cur != dev) {
            const hipError_t r = hipSetDevice(cur);
            if (e == hipSuccess) e = r;
        }
        if (e != hipSuccess) {
            (void)aux_destroy(a);  // the creation error is the one reported
            return e;
        }
        t_aux[dev] = a;
    }
    *out = t_aux[dev];
    return hipSuccess;
}

// Scratch of fwpkm_forward_seq_static, for callers that cannot allocate:
// a file-scope device array, one copy per GPU the library runs on, held
// until the process ends.  Host code never uses the array's name as an
// address (on the host it is only a handle): static_scratch() resolves each
// device's copy once, with that device current, and every later use goes
// through the resolved pointer.
constexpr size_t kStaticScratchBytes = FWPKM_STATIC_SCRATCH_BYTES;
static __device__ __align__(256) unsigned char scratch[kStaticScratchBytes];

hipError_t static_scratch(hipStream_t caller, void** out) {
    static std::mutex mu;
    static void* per_dev[64] = {};
    int dev = 0;
    hipError_t e = stream_device(caller, &dev);
    if (e != hipSuccess) return e;
    if (dev < 0 || dev >= 64) return hipErrorInvalidDevice;
    std::lock_guard<std::mutex> lk(mu);
    if (!per_dev[dev]) {
        int cur = 0;
        if ((e = hipGetDevice(&cur)) != hipSuccess) return e;
        if (cur != dev && (e = hipSetDevice(dev)) != hipSuccess) return e;
        void* p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (cur != dev) {
            const hipError_t r = hipSetDevice(cur);
            if (e == hipSuccess) e = r;
        }
        if (e != hipSuccess) return e;
        if (!p) return hipErrorInvalidSymbol;
        per_dev[dev] = p;
    }
    *out = per_dev[dev];
    return hipSuccess;
}

// Environment overrides for tests, sweeps and profiling, read only while
// FWPKM_DEBUG=1 (otherwise NULL): FWPKM_SINGLE_STREAM, FWPKM_SCORE_PATH,
// FWPKM_KGRAD_SPLIT, FWPKM_DECODE.
const char* debug_env(const char* name) {
    const char* on = std::getenv("FWPKM_DEBUG");
    if (!on || std::strcmp(on, "1") != 0) return nullptr;
    return std::getenv(name);
}

// Chunks with fewer reads (sequences x tokens x heads x k) than this run
// their selection and sort on forward_seq's selection stream.
constexpr int64_t kApartReads = int64_t{1} << 19;

struct Plan {
    int n, H, dq, dh, dv, kh, k, C, store, es;
    int64_t N;
    float eps, lr_v, lr_k, zeps;
    int look, znorm, addr, gate, dot;
    CandTable cand;
    int ncand;
    int sort_passes;
};

int make_plan(const fwpkm_cfg* c, Plan* p) {
    if (!c) return fail(FWPKM_EINVAL, "cfg is NULL");
    if (c->n < 1) return fail(FWPKM_EINVAL, "n must be >= 1 (got %d)", c->n);
    if (static_cast<int64_t>(c->n) * c->n > 2147483647LL) return fail(FWPKM_EINVAL, "n*n overflows int32");
    if (c->heads < 1) return fail(FWPKM_EINVAL, "heads must be >= 1 (got %d)", c->heads);
    if (c->d_q < 2 || (c->d_q & 1)) return fail(FWPKM_EINVAL, "d_q must be even and >= 2 (got %d)", c->d_q);
    if (c->d_v < 1) return fail(FWPKM_EINVAL, "d_v must be >= 1 (got %d)", c->d_v);
    if (c->k_half < 1 || c->k_half > c->n) return fail(FWPKM_EINVAL, "k_half must be in [1, n] (got %d)", c->k_half);
    if (c->k < 1 || static_cast<int64_t>(c->k) > static_cast<int64_t>(c->k_half) * c->k_half)
        return fail(FWPKM_EINVAL, "k must be in [1, k_half^2] (got %d)", c->k);
    if (c->chunk < 1) return fail(FWPKM_EINVAL, "chunk must be >= 1 (got %d)", c->chunk);
    if (c->store != FWPKM_F32 && c->store != FWPKM_BF16) return fail(FWPKM_EINVAL, "store must be FWPKM_F32 or FWPKM_BF16");
    if (c->score != FWPKM_SCORE_IDW && c->score != FWPKM_SCORE_DOT)
        return fail(FWPKM_EINVAL, "score must be FWPKM_SCORE_IDW or FWPKM_SCORE_DOT");
    if (!(c->idw_eps > 0.f) || !std::isfinite(c->idw_eps)) return fail(FWPKM_EINVAL, "idw_eps must be finite and > 0");
    if (!std::isfinite(c->lr_v) || !std::isfinite(c->lr_k)) return fail(FWPKM_EINVAL, "lr_v and lr_k must be finite");
    if (!(c->znorm_eps >= 0.f) || !std::isfinite(c->znorm_eps)) return fail(FWPKM_EINVAL, "znorm_eps must be finite and >= 0");
    // limits of this GPU path
    if (c->n < 16 || c->n > 1024 || (c->n % 16))
        return fail(FWPKM_EUNSUPPORTED, "GPU path needs 16 <= n <= 1024 and n %% 16 == 0 (got %d)", c->n);
    const int dh = c->d_q / 2;
    if (dh != 32 && dh != 64 && dh != 128 && dh != 256)
        return fail(FWPKM_EUNSUPPORTED, "GPU path needs d_q/2 in {32, 64, 128, 256} (got %d)", dh);
    if (c->d_v != 64 && c->d_v != 128 && c->d_v != 256 && c->d_v != 512)
        return fail(FWPKM_EUNSUPPORTED, "GPU path needs d_v in {64, 128, 256, 512} (got %d)", c->d_v);
    if (c->k_half > kMaxKHalf) return fail(FWPKM_EUNSUPPORTED, "GPU path needs k_half <= %d", kMaxKHalf);
    if (c->k > kMaxK) return fail(FWPKM_EUNSUPPORTED, "GPU path needs k <= %d", kMaxK);
    if (static_cast<int64_t>(c->heads) * c->k > 256) return fail(FWPKM_EUNSUPPORTED, "GPU path needs heads*k <= 256");

    p->n = c->n; p->H = c->heads; p->dq = c->d_q; p->dh = dh; p->dv = c->d_v;
    p->kh = c->k_half; p->k = c->k; p->C = c->chunk; p->store = c->store;
    p->es = (c->store == FWPKM_BF16) ? 2 : 4;
    p->N = static_cast<int64_t>(c->n) * c->n;
    p->eps = c->idw_eps; p->lr_v = c->lr_v; p->lr_k = c->lr_k; p->zeps = c->znorm_eps;
    p->look = c->lookahead != 0; p->znorm = c->znorm != 0; p->addr = c->use_addr != 0;
    p->gate = c->gate_weight != 0; p->dot = c->score == FWPKM_SCORE_DOT;
    // product candidates: ranks (a, b) of the two sorted lists with (a+1)(b+1) <= k
    int m = 0;
    std::memset(&p->cand, 0, sizeof p->cand);
    for (int a = 0; a < p->kh; ++a)
        for (int b = 0; b < p->kh; ++b)
            if (static_cast<int64_t>(a + 1) * (b + 1) <= p->k) {
                if (m >= kMaxCand) return fail(FWPKM_EUNSUPPORTED, "too many product candidates for k=%d", p->k);
                p->cand.ab[m++] = static_cast<uint16_t>(a * 64 + b);
            }
    p->ncand = m;
    int bits = 1;
    while ((int64_t{1} << bits) <= p->N) ++bits;  // keys 0..N inclusive (N = sentinel)
    p->sort_passes = (bits + 7) / 8;
    return FWPKM_OK;
}

// Whole-row scoring (k_rows + reductions over the stored rows) for chunks
// whose 64-token tiles cannot give every compute unit a workgroup (decode,
// a single long sequence), as long as the rows fit kRowBytesCap.
constexpr size_t kRowBytesCap = static_cast<size_t>(512) << 20;

size_t row_bytes(const Plan& p, int B, int Tc) {
    return static_cast<size_t>(B) * p.H * 2 * static_cast<size_t>(Tc) * p.n * 4;
}

// FWPKM_SCORE_PATH = "sweep" or "rows" overrides the choice (both compute
// the same selection; the statistics differ only in summation order).
int score_path_override() {
    const char* e = debug_env("FWPKM_SCORE_PATH");
    if (!e) return 0;
    if (std::strcmp(e, "sweep") == 0) return 1;
    if (std::strcmp(e, "rows") == 0) return 2;
    return 0;
}

bool use_rows(const Plan& p, int B, int Tc) {
    const int ov = score_path_override();
    if (ov == 1) return false;
    if (ov == 2) return row_bytes(p, B, Tc) <= kRowBytesCap || Tc <= kRowTok;
    if (Tc <= kRowTok) return true;
    const long long wgs = static_cast<long long>(B) * p.H * 2 * ((Tc + kScoreTokMin - 1) / kScoreTokMin);
    return wgs < device_cus() && row_bytes(p, B, Tc) <= kRowBytesCap;
}

// Longest chunk of at most T tokens scored by whole rows: both conditions of
// use_rows are monotone in Tc, so the chunks that use rows are 1..rows_max.
int rows_max(const Plan& p, int B, int T) {
    const long long m = static_cast<long long>(B) * p.H * 2;
    const int ov = score_path_override();
    if (ov == 1) return 0;
    const long long by_tiles = ov == 2 ? T : 64 * ((device_cus() - 1) / m);  // m * ceil(Tc/64) < CUs
    const long long by_bytes = static_cast<long long>(kRowBytesCap / (static_cast<size_t>(m) * p.n * 4));
    const long long tmax = std::min<long long>(T, std::min(by_tiles, by_bytes));
    return static_cast<int>(std::max<long long>(tmax, std::min(T, kRowTok)));
}

// FWPKM_KGRAD_SPLIT = <s> fixes the key step's token split at s (capped by
// the chunk's 32-token blocks) in place of the per-sequence rule.
int kgrad_split_override() {
    const char* e = debug_env("FWPKM_KGRAD_SPLIT");
    return e ? std::max(0, std::atoi(e)) : 0;
}

// Token tile of the usage partials for a chunk.
int stat_tile(const Plan& p, int B, int Tc) {
    return use_rows(p, B, Tc) ? kScoreTokMin : score_tile(B, p.H, Tc, p.dot != 0);
}

constexpr size_t kAlign = 256;
size_t up(size_t x) { return (x + kAlign - 1) / kAlign * kAlign; }

// Workspace carve-up for B sequences of Tt tokens per step.
struct Layout {
    size_t idx, w, idx2, w2, knorm, qn, cand, cnt, erow, r, Z, M, m, part, lp, qT, kpart, ph, pt, pts, phe;
    // radix sort ping-pong buffers and per-tile digit counts, [1] only with iw_copies = 2
    size_t k0[2], v0[2], k1[2], v1[2], counts[2];
    size_t total;
};

// iw_copies = 2 double-buffers the slot/weight lists across chunks (forward_seq).
Layout layout(const Plan& p, int B, int Tt, bool with_iw, bool with_update, int iw_copies = 1) {
    Layout L{};
    size_t off = 0;
    auto take = [&](size_t bytes) {
        const size_t at = off;
        off += up(bytes);
        return at;
    };
    const size_t Bs = static_cast<size_t>(B), T = static_cast<size_t>(Tt);
    const size_t ntiles = (T + kScoreTokMin - 1) / kScoreTokMin;
    L.knorm = take(Bs * p.H * 2 * p.n * 4);
    L.qn = take(Bs * p.H * 2 * T * 4);
    if (with_iw) {
        L.idx = take(Bs * T * p.H * p.k * 4);
        L.w = take(Bs * T * p.H * p.k * 4);
        if (iw_copies > 1) {
            L.idx2 = take(Bs * T * p.H * p.k * 4);
            L.w2 = take(Bs * T * p.H * p.k * 4);
        }
        L.cand = take(Bs * p.H * 2 * T * static_cast<size_t>(score_cap(p.kh)) * 8);
        L.cnt = take(Bs * p.H * 2 * T * 4);
    }
    L.erow = take(row_bytes(p, B, rows_max(p, B, Tt)));
    if (with_update) {
        const size_t M = T * p.H * p.k;
        const size_t tiles = (M + kSortTileSmall - 1) / kSortTileSmall;  // the most any tile size gives
        // the most pieces any chunk of up to T tokens with targets can need
        // (smaller chunks may use smaller pieces)
        size_t pieces = 1;
        for (int nt = 1; nt <= Tt; ++nt) {
            const int Mn = nt * p.H * p.k, pc = scatter_piece(Mn);
            pieces = std::max(pieces, static_cast<size_t>((Mn + pc - 1) / pc));
        }
        L.r = take(Bs * T * p.dv * 4);
        L.Z = take(Bs * p.H * 2 * T * 4);
        L.M = take(Bs * p.H * 2 * T * 4);
        L.m = take(Bs * p.H * 2 * T * 4);
        L.part = take(Bs * p.H * 2 * ntiles * p.n * 4);
        L.lp = take(Bs * p.H * 2 * p.n * 4);
        L.qT = take(Bs * p.H * 2 * p.dh * ((T + 31) / 32 * 32) * p.es);
        int ksplit = 1;
        for (int nt = 1; nt <= Tt; nt += 32) ksplit = std::max(ksplit, kgrad_split(p.H, p.n, nt, kgrad_split_override(), nullptr));
        L.kpart = ksplit > 1 ? take(kgrad_part_floats(B, p.H, p.n, p.dh, ksplit) * 4) : 0;
        // forward_seq sorts chunk c+1 while chunk c's write still reads its
        // sorted reads, and two chunks' sorts may run at once on different
        // streams: a second set of sort buffers and digit counts, by chunk parity
        for (int set = 0; set < std::min(iw_copies, 2); ++set) {
            L.k0[set] = take(Bs * M * 4);
            L.v0[set] = take(Bs * M * 4);
            L.k1[set] = take(Bs * M * 4);
            L.v1[set] = take(Bs * M * 4);
            L.counts[set] = take(Bs * 256 * std::max<size_t>(tiles, 1) * 4 * p.sort_passes);  // one array per pass
        }
        L.ph = take(Bs * pieces * p.dv * 4);
        L.pt = take(Bs * pieces * p.dv * 4);
        L.pts = take(Bs * pieces * 4);
        L.phe = take(Bs * pieces * 4);
    }
    L.total = off;
    return L;
}

size_t need_retrieve(const Plan& p, int B, int T) { return layout(p, B, T, true, false).total; }
size_t need_update(const Plan& p, int B, int T) { return layout(p, B, T, false, true).total; }
size_t need_forward(const Plan& p, int B, int T) { return layout(p, B, std::min(T, p.C), true, true, 2).total; }

template <class T>
T* at(void* ws, size_t off) {
    return reinterpret_cast<T*>(static_cast<unsigned char*>(ws) + off);
}

int check_ws(void* ws, size_t ws_bytes, size_t need) {
    if (need == 0) return FWPKM_OK;
    if (!ws) return fail(FWPKM_EWORKSPACE, "workspace is NULL (need %zu bytes)", need);
    if (reinterpret_cast<uintptr_t>(ws) % kAlign) return fail(FWPKM_EWORKSPACE, "workspace must be 256-byte aligned");
    if (ws_bytes < need) return fail(FWPKM_EWORKSPACE, "workspace has %zu bytes, needs %zu", ws_bytes, need);
    return FWPKM_OK;
}

#define HIP_TRY(expr)                                                              \
    do {                                                                           \
        hipError_t e_ = (expr);                                                    \
        if (e_ != hipSuccess) return fail(FWPKM_EHIP, "%s: %s", #expr, hipGetErrorString(e_)); \
    } while (0)

hipError_t knorm_launch(const Plan& p, int B, const void* K1, const void* K2, float* knorm, hipStream_t s) {
    TimedLaunch tl(FWPKM_K_KNORM, s);
    KnormArgs a{K1, K2, knorm, B, p.H, p.n, p.dh};
    return launch_knorm(a, p.store, s);
}

// Scoring of Tc tokens (q with per-sequence stride q_bstride elements).
ScoreArgs score_args(const Plan& p, int B, int Tc, const void* q, int64_t q_bstride, const void* K1,
                     const void* K2, const float* knorm, int mode) {
    ScoreArgs a{};
    a.q = q; a.q_bstride = q_bstride; a.K1 = K1; a.K2 = K2; a.knorm = knorm;
    a.B = B; a.Tc = Tc; a.n = p.n; a.H = p.H; a.dh = p.dh; a.kh = p.kh;
    a.eps = p.eps; a.mode = mode; a.cap = score_cap(p.kh); a.dot = p.dot;
    return a;
}

// Selection arguments for the scoring `a` just launched.
SelectArgs select_args(const Plan& p, const ScoreArgs& a, const void* q, int64_t q_bstride, const void* K1,
                       const void* K2, int32_t* idx, float* w, int64_t iw_bstride, int32_t* usage) {
    SelectArgs sa{};
    sa.cand = a.cand; sa.cnt = a.cnt; sa.cap = a.cap;
    sa.q = q; sa.q_bstride = q_bstride; sa.K1 = K1; sa.K2 = K2;
    sa.B = a.B; sa.Tc = a.Tc; sa.n = p.n; sa.H = p.H; sa.dh = p.dh; sa.kh = p.kh; sa.k = p.k; sa.ncand = p.ncand;
    sa.eps = p.eps; sa.idx = idx; sa.w = w; sa.iw_bstride = iw_bstride; sa.cand_ab = p.cand;
    sa.erow = a.erow;
    sa.usage = usage;
    sa.dot = p.dot;
    return sa;
}

// Retrieval's selection of Tc tokens: candidate scoring, then per (token,
// head) top-k' of each half and the product top-k into idx / w.
int select_topk(const Plan& p, const Layout& L, void* ws, int B, int Tc, const void* q, int64_t q_bstride,
                const void* K1, const void* K2, const float* knorm, int32_t* idx, float* w, int64_t iw_bstride,
                bool stats, int32_t* usage, hipStream_t s, hipStream_t s_sel = nullptr, hipEvent_t ev_scored = nullptr) {
    // short chunks (decode, one long sequence): whole rows of e, an exact
    // top-k' of each and statistics by reductions over the rows; otherwise
    // the two-pass sweep with candidate lists.  With `s_sel` (sweep path
    // only) the selection runs there, after the scoring on `s`.
    const bool rows = use_rows(p, B, Tc);
    ScoreArgs a = score_args(p, B, Tc, q, q_bstride, K1, K2, knorm,
                             rows ? kScoreRows : (kScoreSelect | (stats ? kScoreStats : 0)));
    if (rows) a.erow = at<uint32_t>(ws, L.erow);
    a.cand = at<uint64_t>(ws, L.cand);
    a.cnt = at<int32_t>(ws, L.cnt);
    a.qn = at<float>(ws, L.qn);
    if (stats) {
        a.part = at<float>(ws, L.part);
        a.Z = at<float>(ws, L.Z);
        a.M = at<float>(ws, L.M);
    }
    {
        TimedLaunch tl(FWPKM_K_SWEEP_SELECT, s);
        HIP_TRY(launch_score(a, p.store, s));
    }
    SelectArgs sa = select_args(p, a, q, q_bstride, K1, K2, idx, w, iw_bstride, usage);
    if (rows && stats) {
        // whole-row selection also leaves Z (and M); the usage partials
        // follow in the addressing step
        sa.Z = a.Z;
        sa.M = a.M;
    }
    hipStream_t ss = s;
    if (s_sel && s_sel != s && !rows) {
        HIP_TRY(hipEventRecord(ev_scored, s));
        HIP_TRY(hipStreamWaitEvent(s_sel, ev_scored, 0));
        ss = s_sel;
    }
    {
        TimedLaunch tl(FWPKM_K_SELECT, ss);
        HIP_TRY(launch_select(sa, p.store, ss));
    }
    return FWPKM_OK;
}

// Memorisation write of one chunk from idx/w (per-sequence stride iw_bstride),
// residual r [B][Tc][dv], n_tgt tokens with targets, in two parts: the sort
// of every sequence's reads by slot (sort_reads, which returns the buffer
// holding the result), then the value write of sequences [b0, b0 + nb)
// (write_rows).
// `set` picks the buffer set (1 exists only in forward_seq's layout); the
// result is reported as 2 * set + the ping-pong side that holds it.
int sort_reads(const Plan& p, const Layout& L, void* ws, int B, int n_tgt, const int32_t* idx, int64_t iw_bstride,
               int* sorted, hipStream_t s, int set = 0) {
    const int M = n_tgt * p.H * p.k;
    *sorted = 2 * set;
    if (M == 0) return FWPKM_OK;
    const int items = sort_items(B, M);
    const int tiles = (M + 256 * items - 1) / (256 * items);
    uint32_t* kb[2] = {at<uint32_t>(ws, L.k0[set]), at<uint32_t>(ws, L.k1[set])};
    uint32_t* vb[2] = {at<uint32_t>(ws, L.v0[set]), at<uint32_t>(ws, L.v1[set])};
    int cur = 0;
    TimedLaunch tl(FWPKM_K_SORT, s);
    for (int pass = 0; pass < p.sort_passes; ++pass) {
        SortArgs a{};
        a.idx = idx; a.idx_bstride = iw_bstride;
        a.kin = kb[cur]; a.vin = vb[cur];
        a.kout = kb[cur ^ 1]; a.vout = vb[cur ^ 1];
        a.counts = at<uint32_t>(ws, L.counts[set]);
        a.B = B; a.M = M; a.tiles = tiles; a.shift = 8 * pass; a.first = pass == 0;
        a.N = static_cast<uint32_t>(p.N);
        a.items = items;
        // small sorts (a chain of short launches): the scatters count the
        // next pass's digits, so only the first pass has a count launch
        // (one sequence of 512 tokens: 18.1-20.8 -> 17.0-19.0 ms per pass;
        // at 8 sequences the atomics contend and the sort gets slower)
        a.passes = p.sort_passes;
        a.fuse = items == kSortItemsSmall && static_cast<int64_t>(B) * tiles <= kSortFuseTiles;
        a.pass_stride = static_cast<int64_t>(B) * tiles * 256;
        HIP_TRY(launch_sort_pass(a, s));
        cur ^= 1;
    }
    *sorted = 2 * set + cur;
    return FWPKM_OK;
}

int write_rows(const Plan& p, const Layout& L, void* ws, int b0, int nb, int Tc, int n_tgt, const float* w,
               int64_t iw_bstride, void* V, int32_t* n_read, int sorted, hipStream_t s) {
    const int M = n_tgt * p.H * p.k;
    if (M == 0) return FWPKM_OK;
    const int piece = scatter_piece(M);
    const int pieces = (M + piece - 1) / piece;
    const size_t kb = static_cast<size_t>(b0);
    ScatterArgs sa{};
    const int set = sorted >> 1;
    sa.keys = at<uint32_t>(ws, (sorted & 1) ? L.k1[set] : L.k0[set]) + kb * M;
    sa.vals = at<uint32_t>(ws, (sorted & 1) ? L.v1[set] : L.v0[set]) + kb * M;
    sa.w = w + kb * iw_bstride; sa.w_bstride = iw_bstride;
    sa.r = at<float>(ws, L.r) + kb * Tc * p.dv;
    sa.V = static_cast<unsigned char*>(V) + kb * static_cast<size_t>(p.N) * p.dv * p.es;
    sa.n_read = n_read ? n_read + kb * static_cast<size_t>(p.N) : nullptr;
    sa.ph = at<float>(ws, L.ph) + kb * pieces * p.dv; sa.pt = at<float>(ws, L.pt) + kb * pieces * p.dv;
    sa.pt_start = at<int32_t>(ws, L.pts) + kb * pieces; sa.ph_end = at<int32_t>(ws, L.phe) + kb * pieces;
    sa.B = nb; sa.M = M; sa.pieces = pieces; sa.piece = piece; sa.H = p.H; sa.k = p.k; sa.dv = p.dv; sa.Tc = Tc;
    sa.N = static_cast<uint32_t>(p.N); sa.lr = p.lr_v; sa.inv_h = 1.f / static_cast<float>(p.H);
    TimedLaunch tl(FWPKM_K_SCATTER, s);
    HIP_TRY(launch_scatter(sa, p.store, s));
    return FWPKM_OK;
}

int memorise(const Plan& p, const Layout& L, void* ws, int B, int Tc, int n_tgt, const int32_t* idx,
             const float* w, int64_t iw_bstride, void* V, int32_t* n_read, hipStream_t s) {
    if (n_read) {
        TimedLaunch tl(FWPKM_K_FILL, s);
        HIP_TRY(launch_fill_i32(n_read, static_cast<int64_t>(B) * p.N, 0, s));
    }
    int sorted = 0;
    int rc = sort_reads(p, L, ws, B, n_tgt, idx, iw_bstride, &sorted, s);
    if (rc) return rc;
    return write_rows(p, L, ws, 0, B, Tc, n_tgt, w, iw_bstride, V, n_read, sorted, s);
}

// Addressing step of one chunk.  With `have_stats` the retrieval already left
// ||q||^2 and Z (and M) in the workspace, and on the sweep path the usage
// partial sums too (on the rows path they are taken here from the stored
// rows); otherwise a stats scoring pass computes all of them first.
// knorm holds ||K_i||^2 of the current codebooks; the key step rewrites it.
// The transposed queries of the key step (written by the row statistic's
// launch).
QtArgs qt_args(const Plan& p, const Layout& L, void* ws, int B, int Tc, const void* q, int64_t q_bstride) {
    return QtArgs{q, q_bstride, at<void>(ws, L.qT), B, Tc, (Tc + 31) / 32 * 32, p.H, p.dh};
}

int address(const Plan& p, const Layout& L, void* ws, int B, int Tc, const void* q, int64_t q_bstride,
            void* K1, void* K2, bool have_stats, float* knorm, hipStream_t s, hipEvent_t before_kstep = nullptr) {
    const bool rows = use_rows(p, B, Tc);
    if (!have_stats) {
        ScoreArgs a = score_args(p, B, Tc, q, q_bstride, K1, K2, knorm, rows ? kScoreRows : kScoreStats);
        a.qn = at<float>(ws, L.qn);
        a.part = at<float>(ws, L.part);
        a.Z = at<float>(ws, L.Z);
        a.M = at<float>(ws, L.M);
        if (rows) a.erow = at<uint32_t>(ws, L.erow);
        TimedLaunch tl(FWPKM_K_SWEEP_STATS, s);
        HIP_TRY(launch_score(a, p.store, s));
        if (rows) HIP_TRY(launch_row_stats(a, 0, p.store, s));
    }
    if (have_stats && rows) {
        // the selection left Z (and M): the per-tile usage partials
        ScoreArgs ca = score_args(p, B, Tc, q, q_bstride, K1, K2, knorm, kScoreRows);
        ca.erow = at<uint32_t>(ws, L.erow);
        ca.part = at<float>(ws, L.part);
        ca.Z = at<float>(ws, L.Z);
        ca.M = at<float>(ws, L.M);
        TimedLaunch tl(FWPKM_K_PBAR, s);
        HIP_TRY(launch_row_stats(ca, 2, p.store, s));
    }
    // the row statistic forms ln pbar from the usage partials itself and
    // leaves it for the key step
    ScoreArgs ra = score_args(p, B, Tc, q, q_bstride, K1, K2, knorm, kScoreRowStat);
    ra.lp = at<float>(ws, L.lp);
    ra.part = at<float>(ws, L.part);
    {
        const int tile = stat_tile(p, B, Tc);
        ra.pbar_ntiles = (Tc + tile - 1) / tile;
    }
    ra.Z = at<float>(ws, L.Z);
    ra.M = at<float>(ws, L.M);
    ra.m = at<float>(ws, L.m);
    // fp32 storage: the transposed queries the key step reads, extra
    // workgroups of the row statistic's launch on the stored-score path, a
    // launch of their own after a rescoring statistic (which has just brought
    // the queries into the last-level cache); bf16 storage: none (the key
    // step reads its query tiles transposed from LDS)
    const bool want_qt = p.store == kF32;
    const QtArgs qa = qt_args(p, L, ws, B, Tc, q, q_bstride);
    {
        TimedLaunch tl(FWPKM_K_SWEEP_ROWSTAT, s);
        if (rows) {
            if (want_qt) ra.qt = qa;
            ra.erow = at<uint32_t>(ws, L.erow);
            HIP_TRY(launch_row_stats(ra, 1, p.store, s));
        } else {
            HIP_TRY(launch_score(ra, p.store, s));
        }
    }
    if (!rows && want_qt) {
        TimedLaunch tl(FWPKM_K_QT, s);
        HIP_TRY(launch_qt(qa, p.store, s));
    }
    const int Tp = (Tc + 31) / 32 * 32;
    KgradArgs ka{};
    ka.q = q; ka.q_bstride = q_bstride; ka.qT = at<void>(ws, L.qT); ka.Tp = Tp;
    ka.K1 = K1; ka.K2 = K2; ka.knorm = knorm;
    ka.qn = at<float>(ws, L.qn); ka.Z = at<float>(ws, L.Z); ka.m = at<float>(ws, L.m); ka.lp = at<float>(ws, L.lp);
    ka.M = at<float>(ws, L.M); ka.dot = p.dot;
    ka.B = B; ka.Tc = Tc; ka.n = p.n; ka.H = p.H; ka.dh = p.dh; ka.eps = p.eps; ka.lr = p.lr_k;
    ka.split = kgrad_split(p.H, p.n, Tc, kgrad_split_override(), &ka.per);
    ka.part = ka.split > 1 ? at<float>(ws, L.kpart) : nullptr;
    // the key step rewrites K1/K2, which a selection on another stream may still read
    if (before_kstep) HIP_TRY(hipStreamWaitEvent(s, before_kstep, 0));
    {
        TimedLaunch tl(FWPKM_K_KGRAD, s);
        HIP_TRY(launch_kgrad(ka, p.store, s));
    }
    return FWPKM_OK;
}

// Streaming state carve-up: sub-key norms and the pending chunk, C token
// slots per sequence.
struct StreamLayout {
    size_t knorm, q, g, tgt, idx, w, vhat;
    size_t total;
};

StreamLayout stream_layout(const Plan& p, int B) {
    StreamLayout S{};
    size_t off = 0;
    auto take = [&](size_t bytes) {
        const size_t at = off;
        off += up(bytes);
        return at;
    };
    const size_t Bs = static_cast<size_t>(B), C = static_cast<size_t>(p.C);
    S.knorm = take(Bs * p.H * 2 * p.n * 4);
    S.q = take(Bs * C * p.H * p.dq * p.es);
    S.g = take(Bs * C * 4);
    S.tgt = take(Bs * C * p.dv * p.es);
    S.idx = take(Bs * C * p.H * p.k * 4);
    S.w = take(Bs * C * p.H * p.k * 4);
    S.vhat = take(Bs * C * p.dv * 4);
    S.total = off;
    return S;
}

size_t need_stream(const Plan& p, int B) {
    return std::max(need_retrieve(p, B, p.C), need_update(p, B, p.C));
}

// The write of the pending chunk's first Tc tokens, n_tgt of them with
// targets: residual, memorisation and addressing, as fwpkm_chunk_update.
int stream_fire(const Plan& p, const StreamLayout& S, void* st, int B, int Tc, int n_tgt, void* K1, void* K2,
                void* V, void* ws, hipStream_t s) {
    const Layout L = layout(p, B, Tc, false, true);
    const int64_t C = p.C;
    if (n_tgt > 0) {
        ResidArgs ra{at<float>(st, S.vhat), at<float>(st, S.g), at<void>(st, S.tgt), at<float>(ws, L.r),
                     C * p.dv, C, C * p.dv, B, Tc, n_tgt, p.dv, p.znorm, p.zeps, p.gate};
        TimedLaunch tl(FWPKM_K_RESID, s);
        HIP_TRY(launch_resid(ra, p.store, s));
    }
    int rc = memorise(p, L, ws, B, Tc, n_tgt, at<int32_t>(st, S.idx), at<float>(st, S.w), C * p.H * p.k, V, nullptr, s);
    if (rc) return rc;
    if (p.addr) {
        rc = address(p, L, ws, B, Tc, at<void>(st, S.q), C * p.H * p.dq, K1, K2, false, at<float>(st, S.knorm), s);
        if (rc) return rc;
    }
    return FWPKM_OK;
}

// Retrieval of tokens [j, j + seg) of this call (T tokens per sequence)
// into the pending slots [pend, pend + seg), with the copies of q, g and the
// targets that the chunk's write will need.
// FWPKM_DECODE=unfused keeps decode's selection and read as two launches (the
// tests compare the two forms).
bool fused_decode_off() {
    const char* e = debug_env("FWPKM_DECODE");
    return e && std::strcmp(e, "unfused") == 0;
}

int stream_retrieve(const Plan& p, const StreamLayout& S, void* st, int B, int T, int j, int seg, int pend,
                    const void* q, const void* v, const float* g, const void* K1, const void* K2, const void* V,
                    float* o, float* vhat, int32_t* usage, void* ws, hipStream_t s) {
    const Layout L = layout(p, B, seg, true, false);
    const int64_t C = p.C;
    const size_t qrow = static_cast<size_t>(p.H) * p.dq * p.es, vrow = static_cast<size_t>(p.dv) * p.es;
    const auto* qb = static_cast<const unsigned char*>(q);
    const auto* vb = static_cast<const unsigned char*>(v);
    auto* sq = at<unsigned char>(st, S.q);
    auto* stg = at<unsigned char>(st, S.tgt);
    const int64_t iwb = C * p.H * p.k;
    int32_t* idx = at<int32_t>(st, S.idx) + static_cast<size_t>(pend) * p.H * p.k;
    float* w = at<float>(st, S.w) + static_cast<size_t>(pend) * p.H * p.k;
    const void* qj = qb + j * qrow;
    const int64_t qbs = static_cast<int64_t>(T) * p.H * p.dq;
    // few tokens scored by whole rows: selection and read fused per token
    const bool fused = use_rows(p, B, seg) && select_gather_fits(p.H, p.k) &&
                       static_cast<int64_t>(B) * seg < kGatherSplitBelow && !fused_decode_off();
    SelectArgs sa{};
    if (fused) {
        ScoreArgs a = score_args(p, B, seg, qj, qbs, K1, K2, at<float>(st, S.knorm), kScoreRows);
        a.erow = at<uint32_t>(ws, L.erow);
        a.cand = at<uint64_t>(ws, L.cand);
        a.cnt = at<int32_t>(ws, L.cnt);
        a.qn = at<float>(ws, L.qn);
        {
            TimedLaunch tl(FWPKM_K_SWEEP_SELECT, s);
            HIP_TRY(launch_score(a, p.store, s));
        }
        sa = select_args(p, a, qj, qbs, K1, K2, idx, w, iwb, usage);
    } else {
        int rc = select_topk(p, L, ws, B, seg, qj, qbs, K1, K2, at<float>(st, S.knorm), idx, w, iwb, false, usage, s);
        if (rc) return rc;
    }
    GatherArgs ga{};
    ga.V = V; ga.idx = idx; ga.w = w; ga.iw_bstride = iwb;
    ga.v = vb + j * vrow; ga.v_bstride = static_cast<int64_t>(T) * p.dv;
    ga.g = g + j; ga.g_bstride = T;
    ga.o = o + static_cast<size_t>(j) * p.dv;
    ga.vhat = vhat ? vhat + static_cast<size_t>(j) * p.dv : nullptr;
    ga.o_bstride = static_cast<int64_t>(T) * p.dv;
    ga.vhat2 = at<float>(st, S.vhat) + static_cast<size_t>(pend) * p.dv; ga.vhat2_bstride = C * p.dv;
    // the token's q, g and (as a target) v into the pending chunk
    ga.q = qb + j * qrow; ga.q_bstride = static_cast<int64_t>(T) * p.H * p.dq; ga.qrow = p.H * p.dq;
    ga.pq = sq + pend * qrow; ga.pq_bstride = C * p.H * p.dq;
    ga.pg = at<float>(st, S.g) + pend; ga.pg_bstride = C;
    // v of token t is the target of pending slot pend + t, or with lookahead
    // of the slot before it (none for the first token of a chunk)
    ga.ptgt = stg; ga.ptgt_bstride = C * p.dv;
    ga.ptgt_shift = p.look ? pend - 1 : pend;
    ga.B = B; ga.Tc = seg; ga.H = p.H; ga.k = p.k; ga.dv = p.dv; ga.N = p.N;
    if (fused) {
        TimedLaunch tl(FWPKM_K_SELECT, s);
        HIP_TRY(launch_select_gather(sa, ga, p.store, s));
    } else {
        TimedLaunch tl(FWPKM_K_GATHER, s);
        HIP_TRY(launch_gather(ga, p.store, s));
    }
    return FWPKM_OK;
}

int stream_args(const fwpkm_cfg* cfg, int32_t B, fwpkm_stream_pos* pos, Plan* p) {
    int rc = make_plan(cfg, p);
    if (rc) return rc;
    if (B < 0) return fail(FWPKM_EINVAL, "B must be >= 0");
    if (!pos) return fail(FWPKM_EINVAL, "pos is NULL");
    if (pos->pending < 0 || pos->pending > p->C)
        return fail(FWPKM_EINVAL, "pos->pending must be in [0, chunk] (got %d)", pos->pending);
    if (static_cast<int64_t>(B) * p->C * p->H * p->k > 2147483647LL)
        return fail(FWPKM_EUNSUPPORTED, "B*C*heads*k too large");
    return FWPKM_OK;
}

int check_state(const void* state) {
    if (!state) return fail(FWPKM_EINVAL, "state is NULL");
    if (reinterpret_cast<uintptr_t>(state) % kAlign) return fail(FWPKM_EINVAL, "state must be 256-byte aligned");
    return FWPKM_OK;
}

}  // namespace

extern "C" {

int32_t fwpkm_abi_version(void) { return FWPKM_ABI_VERSION; }

const char* fwpkm_last_error(void) { return g_err.c_str(); }

int fwpkm_workspace_bytes(const fwpkm_cfg* cfg, int32_t B, int32_t T, size_t* bytes) {
    Plan p;
    int rc = make_plan(cfg, &p);
    if (rc) return rc;
    if (B < 0 || T < 0) return fail(FWPKM_EINVAL, "B and T must be >= 0");
    if (!bytes) return fail(FWPKM_EINVAL, "bytes is NULL");
    if (B == 0 || T == 0) {
        *bytes = 0;
        return ok();
    }
    *bytes = std::max(need_retrieve(p, B, T), std::max(need_update(p, B, T), need_forward(p, B, T)));
    return ok();
}

int fwpkm_retrieve(const fwpkm_cfg* cfg, int32_t B, int32_t T, const void* q, const void* v, const float* g,
                   const void* K1, const void* K2, const void* V, float* o, float* vhat, int32_t* idx, float* w,
                   void* ws, size_t ws_bytes, void* stream) {
    Plan p;
    int rc = make_plan(cfg, &p);
    if (rc) return rc;
    if (B < 0 || T < 0) return fail(FWPKM_EINVAL, "B and T must be >= 0");
    if (static_cast<int64_t>(B) * T * p.H * p.k > 2147483647LL) return fail(FWPKM_EUNSUPPORTED, "B*T*heads*k too large");
    if (B == 0 || T == 0) return ok();
    if (!q || !v || !g || !K1 || !K2 || !V || !o) return fail(FWPKM_EINVAL, "q, v, g, K1, K2, V and o are required");
    const Layout L = layout(p, B, T, true, false);
    rc = check_ws(ws, ws_bytes, L.total);
    if (rc) return rc;
    hipStream_t s = static_cast<hipStream_t>(stream);
    HIP_TRY(knorm_launch(p, B, K1, K2, at<float>(ws, L.knorm), s));
    int32_t* ii = idx ? idx : at<int32_t>(ws, L.idx);
    float* ww = w ? w : at<float>(ws, L.w);
    const int64_t iwb = static_cast<int64_t>(T) * p.H * p.k;
    rc = select_topk(p, L, ws, B, T, q, static_cast<int64_t>(T) * p.H * p.dq, K1, K2, at<float>(ws, L.knorm), ii, ww,
                     iwb, false, nullptr, s);
    if (rc) return rc;
    GatherArgs ga{};
    ga.V = V; ga.idx = ii; ga.w = ww; ga.iw_bstride = iwb;
    ga.v = v; ga.v_bstride = static_cast<int64_t>(T) * p.dv;
    ga.g = g; ga.g_bstride = T;
    ga.o = o; ga.vhat = vhat; ga.o_bstride = static_cast<int64_t>(T) * p.dv;
    ga.B = B; ga.Tc = T; ga.H = p.H; ga.k = p.k; ga.dv = p.dv; ga.N = p.N;
    {
        TimedLaunch tl(FWPKM_K_GATHER, s);
        HIP_TRY(launch_gather(ga, p.store, s));
    }
    return ok();
}

int fwpkm_chunk_update(const fwpkm_cfg* cfg, int32_t B, int32_t Tc, int32_t n_tgt, const void* q, const float* g,
                       const void* tgt, const int32_t* idx, const float* w, const float* vhat, void* K1, void* K2,
                       void* V, int32_t* n_read, void* ws, size_t ws_bytes, void* stream) {
    Plan p;
    int rc = make_plan(cfg, &p);
    if (rc) return rc;
    if (B < 0 || Tc < 0) return fail(FWPKM_EINVAL, "B and Tc must be >= 0");
    if (n_tgt < 0 || n_tgt > Tc) return fail(FWPKM_EINVAL, "n_tgt must be in [0, Tc] (got %d, Tc=%d)", n_tgt, Tc);
    if (static_cast<int64_t>(B) * Tc * p.H * p.k > 2147483647LL) return fail(FWPKM_EUNSUPPORTED, "B*Tc*heads*k too large");
    if (B == 0 || Tc == 0) return ok();
    if (!q || !g || !idx || !w || !vhat || !K1 || !K2 || !V)
        return fail(FWPKM_EINVAL, "q, g, idx, w, vhat, K1, K2 and V are required");
    if (n_tgt > 0 && !tgt) return fail(FWPKM_EINVAL, "tgt is required when n_tgt > 0");
    const Layout L = layout(p, B, Tc, false, true);
    rc = check_ws(ws, ws_bytes, L.total);
    if (rc) return rc;
    hipStream_t s = static_cast<hipStream_t>(stream);
    HIP_TRY(knorm_launch(p, B, K1, K2, at<float>(ws, L.knorm), s));
    if (n_tgt > 0) {
        ResidArgs ra{vhat, g, tgt, at<float>(ws, L.r), static_cast<int64_t>(Tc) * p.dv, Tc,
                     static_cast<int64_t>(n_tgt) * p.dv, B, Tc, n_tgt, p.dv, p.znorm, p.zeps, p.gate};
        TimedLaunch tl(FWPKM_K_RESID, s);
        HIP_TRY(launch_resid(ra, p.store, s));
    }
    const int64_t iwb = static_cast<int64_t>(Tc) * p.H * p.k;
    rc = memorise(p, L, ws, B, Tc, n_tgt, idx, w, iwb, V, n_read, s);
    if (rc) return rc;
    if (p.addr) {
        rc = address(p, L, ws, B, Tc, q, static_cast<int64_t>(Tc) * p.H * p.dq, K1, K2, false, at<float>(ws, L.knorm),
                     s);
        if (rc) return rc;
    }
    return ok();
}

}  // extern "C"

namespace {

// Gradient outputs of a replayed pass (fwpkm_forward_seq_backward).
struct SeqGrad {
    const float* dO;
    float* dq;
    float* dv;
    float* dg;
};

int forward_seq_impl(const fwpkm_cfg* cfg, int32_t B, int32_t T, int32_t passes, const void* q, const void* v,
                     const float* g, const void* v_next, void* K1, void* K2, void* V, float* o, float* vhat,
                     int32_t* usage, const SeqGrad* grad, void* ws, size_t ws_bytes, void* stream,
                     bool use_static = false) {
    Plan p;
    int rc = make_plan(cfg, &p);
    if (rc) return rc;
    if (B < 0 || T < 0) return fail(FWPKM_EINVAL, "B and T must be >= 0");
    if (passes < 1) return fail(FWPKM_EINVAL, "passes must be >= 1 (got %d)", passes);
    if (B == 0 || T == 0) return ok();
    if (!q || !v || !g || !K1 || !K2 || !V || (!o && !grad))
        return fail(FWPKM_EINVAL, "q, v, g, K1, K2, V and o are required");
    if (grad && (!grad->dO || !grad->dq || !grad->dv || !grad->dg))
        return fail(FWPKM_EINVAL, "dO, dq, dv and dg are required");
    const int Cm = std::min(T, p.C);
    if (static_cast<int64_t>(B) * Cm * p.H * p.k > 2147483647LL) return fail(FWPKM_EUNSUPPORTED, "B*C*heads*k too large");
    const Layout L = layout(p, B, Cm, true, true, 2);
    hipStream_t s = static_cast<hipStream_t>(stream);
    if (use_static) {
        if (L.total > kStaticScratchBytes)
            return fail(FWPKM_EWORKSPACE, "this call needs %zu bytes of scratch; the static scratch holds %zu",
                        L.total, kStaticScratchBytes);
        HIP_TRY(static_scratch(s, &ws));
        ws_bytes = kStaticScratchBytes;
    }
    rc = check_ws(ws, ws_bytes, L.total);
    if (rc) return rc;
    // The key path (scoring, selection, usage statistics, key step) stays on
    // the caller's stream; the value path (sort, gather, value write) of the
    // same chunk runs on a value stream of the library.  They meet at the
    // selection of each chunk.  On the sweep path, chunks of fewer than
    // kApartReads reads move the selection and the sort to a third,
    // selection stream: the selection waits for the scoring, the key step
    // for the selection (which reads K1/K2), so the usage statistics overlap
    // the selection, and the sort leaves the value path.  (On the rows path
    // the statistics use what the selection leaves, so it stays on the key
    // path.)  Measured: 131K-read chunks (B = 8, 4 heads, k = 16, 256
    // tokens) 2.31 -> 2.22 ms per step; at 1M reads (B = 16, 4 heads,
    // k = 32, 512 tokens) the value path already fills HBM and the extra
    // concurrency slows it, 7.99 -> 8.15 ms, so there they stay.  The
    // slot/weight lists and the sort buffers alternate between two sets, so
    // chunk c+1's selection and sort only wait for chunk c-1's write.  With
    // kernel timing on, in fwpkm_forward_seq_static, or with the debug
    // override FWPKM_SINGLE_STREAM=1, everything stays on `stream` (same
    // work, one kernel at a time) and no stream or event of the library is
    // used.
    const char* env_single = debug_env("FWPKM_SINGLE_STREAM");
    // the replay for gradients keeps every kernel in order on one stream:
    // a chunk's gradient reads V and K before that chunk's write
    const bool single =
        use_static || timing().on || (env_single && env_single[0] == '1') || grad != nullptr;
    Aux none;  // no events: every record and wait below is skipped when single
    Aux* ax = &none;
    if (!single) HIP_TRY(aux_streams(s, &ax));
    auto record = [&](hipEvent_t ev, hipStream_t st) { return single ? hipSuccess : hipEventRecord(ev, st); };
    auto wait = [&](hipStream_t st, hipEvent_t ev) { return single ? hipSuccess : hipStreamWaitEvent(st, ev, 0); };
    hipStream_t sv = single ? s : ax->sv;
    hipStream_t sx = single ? s : ax->sx;
    // With two streams the value path of a chunk runs as two half-batch
    // launches of gather + write: between them the key path's kernels find
    // room on the chip (measured: 9.30 -> 8.83 ms per step at B=16); see
    // below for the one exception.
    const int group = single ? B : std::max(1, (B + 1) / 2);
    HIP_TRY(record(ax->ev_start, s));
    HIP_TRY(wait(sv, ax->ev_start));
    HIP_TRY(wait(sx, ax->ev_start));
    HIP_TRY(knorm_launch(p, B, K1, K2, at<float>(ws, L.knorm), s));
    const int64_t qb = static_cast<int64_t>(T) * p.H * p.dq;
    const int64_t vbs = static_cast<int64_t>(T) * p.dv;
    const int nchunks = (T + p.C - 1) / p.C;
    int32_t* idxs[2] = {at<int32_t>(ws, L.idx), at<int32_t>(ws, L.idx2)};
    float* ws_w[2] = {at<float>(ws, L.w), at<float>(ws, L.w2)};
    int64_t step = 0;
    for (int pass = 0; pass < passes; ++pass) {
        const bool last_pass = pass == passes - 1;
        for (int c = 0; c < nchunks; ++c, ++step) {
            const int t0 = c * p.C;
            const int Tc = std::min(p.C, T - t0);
            const unsigned char* qc = static_cast<const unsigned char*>(q) + static_cast<size_t>(t0) * p.H * p.dq * p.es;
            const unsigned char* vc = static_cast<const unsigned char*>(v) + static_cast<size_t>(t0) * p.dv * p.es;
            const int64_t iwb = static_cast<int64_t>(Tc) * p.H * p.k;
            const int buf = static_cast<int>(step & 1);
            int32_t* idx = idxs[buf];
            float* w = ws_w[buf];
            // where this chunk's selection and sort run: apart from the key and
            // value paths on the sweep path of chunks with fewer than
            // kApartReads reads; bigger chunks keep them on those paths
            const int64_t reads = static_cast<int64_t>(B) * Tc * p.H * p.k;
            const bool sel_apart = sx != s && !use_rows(p, B, Tc) && reads < kApartReads;
            hipStream_t ss = sel_apart ? sx : s;
            // these lists and sort buffers were last read by the value write two chunks ago
            if (step >= 2) HIP_TRY(wait(ss, ax->ev_write[buf]));
            // retrieval with the state left by the previous chunk
            rc = select_topk(p, L, ws, B, Tc, qc, qb, K1, K2, at<float>(ws, L.knorm), idx, w, iwb, p.addr, usage, s,
                             sel_apart ? sx : nullptr, ax->ev_scored);
            if (rc) return rc;
            HIP_TRY(record(ax->ev_sel, ss));

            // targets: lookahead pairs t with t+1; the sequence's last token uses v_next or has none
            int n_tgt;
            const void* tgt;
            const void* tgt_last = nullptr;
            if (!p.look) {
                n_tgt = Tc;
                tgt = vc;
            } else {
                tgt = vc + static_cast<size_t>(p.dv) * p.es;
                const bool at_end = t0 + Tc == T;
                if (!at_end) {
                    n_tgt = Tc;
                } else if (v_next) {
                    n_tgt = Tc;
                    tgt_last = v_next;
                } else {
                    n_tgt = Tc - 1;
                }
            }
            // the sort of all reads, then the value path: gather and value
            // write by groups of `group` sequences
            const bool sort_apart = sel_apart;
            hipStream_t so = sort_apart ? sx : sv;
            if (ss != so) HIP_TRY(wait(so, ax->ev_sel));
            int sorted = 0;
            // chunks alternate between two sets of sort buffers (keys, values
            // and digit counts) wherever their sort runs.  A chunk's sort and
            // write touch only its own set, last used by the chunk two before,
            // whose write ev_write[buf] orders first.  Nothing orders the sorts
            // of neighbouring chunks against each other: a pass's short last
            // chunk may sort apart while the chunk before it still sorts or is
            // written on the value stream, so the two must share no buffer.
            rc = sort_reads(p, L, ws, B, n_tgt, idx, iwb, &sorted, so, buf);
            if (rc) return rc;
            if (so != sv) {
                HIP_TRY(record(ax->ev_sorted, so));
                HIP_TRY(wait(sv, ax->ev_sorted));
            }
            // with the selection apart, a half batch of under 4 sequences is
            // too few wavefronts for the write: one launch (measured, 4
            // sequences, 1024 tokens: 1.38 -> 1.36 ms per step; 8 sequences
            // of 256 tokens lose 2.21 -> 2.33 ms the same way)
            const int grp = (sel_apart && group < 4) ? B : group;
            for (int b0 = 0; b0 < B; b0 += grp) {
                const int nb = std::min(grp, B - b0);
                const size_t bo = static_cast<size_t>(b0);
                GatherArgs ga{};
                ga.V = static_cast<unsigned char*>(V) + bo * static_cast<size_t>(p.N) * p.dv * p.es;
                ga.idx = idx + bo * iwb; ga.w = w + bo * iwb; ga.iw_bstride = iwb;
                ga.v = vc + bo * vbs * p.es; ga.v_bstride = vbs;
                ga.g = g + t0 + bo * T; ga.g_bstride = T;
                ga.tgt = static_cast<const unsigned char*>(tgt) + bo * vbs * p.es; ga.tgt_bstride = vbs;
                ga.n_tgt = n_tgt;
                ga.tgt_last = tgt_last ? static_cast<const unsigned char*>(tgt_last) + bo * p.dv * p.es : nullptr;
                ga.tgt_last_bstride = p.dv;
                ga.o = (last_pass && o) ? o + bo * vbs + static_cast<size_t>(t0) * p.dv : nullptr;
                ga.vhat = (last_pass && vhat) ? vhat + bo * vbs + static_cast<size_t>(t0) * p.dv : nullptr;
                ga.o_bstride = vbs;
                ga.r = at<float>(ws, L.r) + bo * Tc * p.dv;
                ga.B = nb; ga.Tc = Tc; ga.H = p.H; ga.k = p.k; ga.dv = p.dv; ga.N = p.N;
                ga.znorm = p.znorm; ga.znorm_eps = p.zeps; ga.gate_w = p.gate;
                ga.keep_b0 = gather_keep_from(nb, Tc, p.H, p.k, p.dv, p.es);
                // rows held raw (more wavefronts per SIMD) in chunks under
                // kApartReads reads, where the value path does not already
                // fill HBM; above, the extra wavefronts only crowd the key
                // path (A/B, the same bits: 131K-read chunks 1.900 -> 1.832
                // ms per step, 262K 1.168 -> 1.160, 1M 7.339 -> 7.41)
                ga.held = reads < kApartReads ? 1 : 0;
                {
                    TimedLaunch tl(FWPKM_K_GATHER, sv);
                    HIP_TRY(launch_gather(ga, p.store, sv));
                }
                if (grad && last_pass) {
                    // gradient of this chunk's o against the state it was read from
                    const size_t t0s = static_cast<size_t>(t0);
                    BackwardArgs ba{};
                    ba.q = qc + bo * qb * p.es; ba.q_bstride = qb;
                    ba.v = ga.v; ba.v_bstride = vbs;
                    ba.g = ga.g; ba.g_bstride = T;
                    ba.idx = ga.idx; ba.w = ga.w; ba.iw_bstride = iwb;
                    ba.K1 = static_cast<const unsigned char*>(K1) + bo * p.H * p.n * p.dh * p.es;
                    ba.K2 = static_cast<const unsigned char*>(K2) + bo * p.H * p.n * p.dh * p.es;
                    ba.V = ga.V;
                    ba.dO = grad->dO + bo * vbs + t0s * p.dv;
                    ba.dq = grad->dq + bo * qb + t0s * p.H * p.dq;
                    ba.dv_out = grad->dv + bo * vbs + t0s * p.dv;
                    ba.dg = grad->dg + bo * T + t0s;
                    ba.B = nb; ba.T = Tc; ba.n = p.n; ba.H = p.H; ba.dh = p.dh; ba.dv = p.dv; ba.k = p.k;
                    ba.N = p.N; ba.eps = p.eps; ba.dot = p.dot;
                    TimedLaunch tl(FWPKM_K_BACKWARD, sv);
                    HIP_TRY(launch_backward(ba, p.store, sv));
                }
                rc = write_rows(p, L, ws, b0, nb, Tc, n_tgt, w, iwb, V, nullptr, sorted, sv);
                if (rc) return rc;
            }
            HIP_TRY(record(ax->ev_write[buf], sv));
            // key path: addressing step of this chunk; the next chunk's
            // scoring rewrites the candidate lists this selection reads
            if (p.addr) {
                rc = address(p, L, ws, B, Tc, qc, qb, K1, K2, true, at<float>(ws, L.knorm), s,
                             sel_apart ? ax->ev_sel : nullptr);
                if (rc) return rc;
            } else if (sel_apart) {
                HIP_TRY(wait(s, ax->ev_sel));
            }
        }
    }
    // join: the caller's stream sees every write
    HIP_TRY(record(ax->ev_end, sv));
    HIP_TRY(wait(s, ax->ev_end));
    return ok();
}

}  // namespace

extern "C" {

int fwpkm_forward_seq(const fwpkm_cfg* cfg, int32_t B, int32_t T, int32_t passes, const void* q, const void* v,
                      const float* g, const void* v_next, void* K1, void* K2, void* V, float* o, float* vhat,
                      void* ws, size_t ws_bytes, void* stream) {
    return forward_seq_impl(cfg, B, T, passes, q, v, g, v_next, K1, K2, V, o, vhat, nullptr, nullptr, ws, ws_bytes,
                            stream);
}

int fwpkm_forward_seq_usage(const fwpkm_cfg* cfg, int32_t B, int32_t T, int32_t passes, const void* q,
                            const void* v, const float* g, const void* v_next, void* K1, void* K2, void* V, float* o,
                            float* vhat, int32_t* usage, void* ws, size_t ws_bytes, void* stream) {
    return forward_seq_impl(cfg, B, T, passes, q, v, g, v_next, K1, K2, V, o, vhat, usage, nullptr, ws, ws_bytes,
                            stream);
}

int fwpkm_forward_seq_backward(const fwpkm_cfg* cfg, int32_t B, int32_t T, int32_t passes, const void* q,
                               const void* v, const float* g, const void* v_next, void* K1, void* K2, void* V,
                               const float* dO, float* dq, float* dv, float* dg, float* o, void* ws, size_t ws_bytes,
                               void* stream) {
    const SeqGrad grad{dO, dq, dv, dg};
    return forward_seq_impl(cfg, B, T, passes, q, v, g, v_next, K1, K2, V, o, nullptr, nullptr, &grad, ws, ws_bytes,
                            stream);
}

int fwpkm_forward_seq_static(const fwpkm_cfg* cfg, int32_t B, int32_t T, int32_t passes, const void* q,
                             const void* v, const float* g, const void* v_next, void* K1, void* K2, void* V,
                             float* o, float* vhat, void* stream) {
    // kernel timing creates its events on demand: not in a call that must not allocate
    if (timing().on) return fail(FWPKM_EINVAL, "fwpkm_forward_seq_static does not run while kernel timing is on");
    return forward_seq_impl(cfg, B, T, passes, q, v, g, v_next, K1, K2, V, o, vhat, nullptr, nullptr, nullptr, 0,
                            stream, true);
}

int fwpkm_release_streams(void) {
    hipError_t first = hipSuccess;
    for (Aux*& a : t_aux)
        if (a) {
            const hipError_t e = aux_destroy(a);
            if (first == hipSuccess) first = e;
            a = nullptr;
        }
    t_aux.clear();
    if (first != hipSuccess) return fail(FWPKM_EHIP, "releasing the library's streams: %s", hipGetErrorString(first));
    return ok();
}

int fwpkm_stream_state_bytes(const fwpkm_cfg* cfg, int32_t B, size_t* bytes) {
    Plan p;
    int rc = make_plan(cfg, &p);
    if (rc) return rc;
    if (B < 0) return fail(FWPKM_EINVAL, "B must be >= 0");
    if (!bytes) return fail(FWPKM_EINVAL, "bytes is NULL");
    *bytes = B == 0 ? 0 : stream_layout(p, B).total;
    return ok();
}

int fwpkm_stream_step(const fwpkm_cfg* cfg, int32_t B, int32_t T, const void* q, const void* v, const float* g,
                      void* K1, void* K2, void* V, float* o, float* vhat, int32_t* usage, void* state,
                      fwpkm_stream_pos* pos, void* ws, size_t ws_bytes, void* stream) {
    Plan p;
    int rc = stream_args(cfg, B, pos, &p);
    if (rc) return rc;
    if (T < 0) return fail(FWPKM_EINVAL, "T must be >= 0");
    if (B == 0 || T == 0) return ok();
    if (!q || !v || !g || !K1 || !K2 || !V || !o) return fail(FWPKM_EINVAL, "q, v, g, K1, K2, V and o are required");
    rc = check_state(state);
    if (rc) return rc;
    rc = check_ws(ws, ws_bytes, need_stream(p, B));
    if (rc) return rc;
    hipStream_t s = static_cast<hipStream_t>(stream);
    const StreamLayout S = stream_layout(p, B);
    if (!pos->norms_valid) {
        HIP_TRY(knorm_launch(p, B, K1, K2, at<float>(state, S.knorm), s));
        pos->norms_valid = 1;
    }
    const size_t vrow = static_cast<size_t>(p.dv) * p.es;
    int pend = pos->pending;
    for (int j = 0; j < T;) {
        if (pend == p.C) {
            // a full chunk; with lookahead token j is its last token's target
            if (p.look) {
                TimedLaunch tl(FWPKM_K_PEND, s);
                HIP_TRY(launch_copy2d(at<unsigned char>(state, S.tgt) + (pend - 1) * vrow,
                                      static_cast<int64_t>(p.C) * vrow,
                                      static_cast<const unsigned char*>(v) + static_cast<size_t>(j) * vrow,
                                      static_cast<int64_t>(T) * vrow, vrow, B, s));
            }
            rc = stream_fire(p, S, state, B, p.C, p.C, K1, K2, V, ws, s);
            if (rc) return rc;
            pend = 0;
        }
        const int seg = std::min(T - j, p.C - pend);
        rc = stream_retrieve(p, S, state, B, T, j, seg, pend, q, v, g, K1, K2, V, o, vhat, usage, ws, s);
        if (rc) return rc;

        pend += seg;
        j += seg;
        pos->pending = pend;
        if (!p.look && pend == p.C) {
            rc = stream_fire(p, S, state, B, p.C, p.C, K1, K2, V, ws, s);
            if (rc) return rc;
            pend = 0;
            pos->pending = 0;
        }
    }
    return ok();
}

int fwpkm_stream_flush(const fwpkm_cfg* cfg, int32_t B, const void* v_next, void* K1, void* K2, void* V,
                       void* state, fwpkm_stream_pos* pos, void* ws, size_t ws_bytes, void* stream) {
    Plan p;
    int rc = stream_args(cfg, B, pos, &p);
    if (rc) return rc;
    if (B == 0 || pos->pending == 0) {
        pos->pending = 0;
        return ok();
    }
    if (!K1 || !K2 || !V) return fail(FWPKM_EINVAL, "K1, K2 and V are required");
    rc = check_state(state);
    if (rc) return rc;
    rc = check_ws(ws, ws_bytes, need_stream(p, B));
    if (rc) return rc;
    hipStream_t s = static_cast<hipStream_t>(stream);
    const StreamLayout S = stream_layout(p, B);
    if (!pos->norms_valid) {
        HIP_TRY(knorm_launch(p, B, K1, K2, at<float>(state, S.knorm), s));
        pos->norms_valid = 1;
    }
    const int pend = pos->pending;
    int n_tgt = pend;
    if (p.look) {
        if (v_next) {
            const size_t vrow = static_cast<size_t>(p.dv) * p.es;
            TimedLaunch tl(FWPKM_K_PEND, s);
            HIP_TRY(launch_copy2d(at<unsigned char>(state, S.tgt) + (pend - 1) * vrow,
                                  static_cast<int64_t>(p.C) * vrow, v_next, static_cast<int64_t>(vrow), vrow, B, s));
        } else {
            n_tgt = pend - 1;
        }
    }
    rc = stream_fire(p, S, state, B, pend, n_tgt, K1, K2, V, ws, s);
    if (rc) return rc;
    pos->pending = 0;
    return ok();
}

int fwpkm_retrieve_backward(const fwpkm_cfg* cfg, int32_t B, int32_t T, const void* q, const void* v, const float* g,
                            const void* K1, const void* K2, const void* V, const int32_t* idx, const float* w,
                            const float* dO, float* dq, float* dv, float* dg, void* stream) {
    Plan p;
    int rc = make_plan(cfg, &p);
    if (rc) return rc;
    if (B < 0 || T < 0) return fail(FWPKM_EINVAL, "B and T must be >= 0");
    if (static_cast<int64_t>(B) * T * p.H * p.k > 2147483647LL) return fail(FWPKM_EUNSUPPORTED, "B*T*heads*k too large");
    if (B == 0 || T == 0) return ok();
    if (!q || !v || !g || !K1 || !K2 || !V || !idx || !w || !dO || !dq || !dv || !dg)
        return fail(FWPKM_EINVAL, "q, v, g, K1, K2, V, idx, w, dO, dq, dv and dg are required");
    BackwardArgs a{q, static_cast<int64_t>(T) * p.H * p.dq, v, static_cast<int64_t>(T) * p.dv, g, T, idx, w,
                   static_cast<int64_t>(T) * p.H * p.k, K1, K2, V, dO, dq, dv, dg, B, T, p.n, p.H, p.dh, p.dv, p.k,
                   p.N, p.eps, p.dot};
    hipStream_t s = static_cast<hipStream_t>(stream);
    TimedLaunch tl(FWPKM_K_BACKWARD, s);
    HIP_TRY(launch_backward(a, p.store, s));
    return ok();
}

int fwpkm_usage_metrics(const fwpkm_cfg* cfg, int32_t B, int32_t* usage, double* metrics, int32_t reset,
                        void* ws, size_t ws_bytes, void* stream) {
    Plan p;
    int rc = make_plan(cfg, &p);
    if (rc) return rc;
    if (B < 0) return fail(FWPKM_EINVAL, "B must be >= 0");
    if (B == 0) return ok();
    if (!usage || !metrics) return fail(FWPKM_EINVAL, "usage and metrics are required");
    rc = check_ws(ws, ws_bytes, static_cast<size_t>(B) * kUsageParts * 32);
    if (rc) return rc;
    hipStream_t s = static_cast<hipStream_t>(stream);
    TimedLaunch tl(FWPKM_K_USAGE, s);
    HIP_TRY(launch_usage_metrics(usage, B, p.N, ws, metrics, reset ? 1 : 0, s));
    return ok();
}

int fwpkm_timing_enable(int32_t on) {
    Timing& t = timing();
    std::lock_guard<std::mutex> lk(t.mu);
    if (on) {
        for (const TimedPair& p : t.pending) {
            t.pool.push_back(p.start);
            t.pool.push_back(p.stop);
        }
        t.pending.clear();
        for (int i = 0; i < FWPKM_K_COUNT; ++i) {
            t.ms[i] = 0.0;
            t.launches[i] = 0;
        }
    }
    t.on = on != 0;
    return ok();
}

int fwpkm_timing_read(int32_t kernel, double* total_ms, int64_t* launches) {
    if (kernel < 0 || kernel >= FWPKM_K_COUNT) return fail(FWPKM_EINVAL, "unknown kernel family %d", kernel);
    if (!total_ms || !launches) return fail(FWPKM_EINVAL, "total_ms and launches are required");
    Timing& t = timing();
    std::lock_guard<std::mutex> lk(t.mu);
    for (const TimedPair& p : t.pending) {
        HIP_TRY(hipEventSynchronize(p.stop));
        float ms = 0.f;
        HIP_TRY(hipEventElapsedTime(&ms, p.start, p.stop));
        t.ms[p.family] += ms;
        t.launches[p.family] += 1;
        t.pool.push_back(p.start);
        t.pool.push_back(p.stop);
    }
    t.pending.clear();
    *total_ms = t.ms[kernel];
    *launches = t.launches[kernel];
    return ok();
}

}  // extern "C"
