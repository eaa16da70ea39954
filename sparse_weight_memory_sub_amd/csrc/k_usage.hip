// k_usage.hip -- slot-usage counts and the addressing metrics.
//
// The addressing metrics ("Fast-weight Product Key Memory", paperlayer.ai
// D.3) are computed from row contributions: the number of accesses c_i to
// each value row i over an interval of tokens.  Coverage is the share of
// rows accessed at least once, collision the share of accesses that land on
// a row accessed more than once, KLD the Kullback-Leibler divergence of the
// access distribution u_i = c_i / S from uniform use of the N rows:
//   KLD = sum_i u_i ln(u_i N) = (1/S) sum_i c_i ln c_i + ln N - ln S.
//
// The counters are filled by the selection kernels (one integer atomic per
// read as its slot id is written: exact, order-free).  The metrics reduce
// each sequence's counters in kUsageParts slices (k_usage_part, fixed-order
// tree per slice, fp64 for the c ln c sum), then add the slices in order
// (k_usage_final): reproducible.  The slices can clear the counters for the
// next interval.
#include "fwpkm_internal.h"

namespace fwpkm {

namespace {

constexpr int kMetricThreads = 256;

// Partial sums of one slice of one sequence's counters: (sum c ln c, reads,
// rows read, reads of rows read more than once), in a fixed order.
struct UsagePart {
    double cl;
    unsigned long long tot, nz, comp;
};

__global__ __launch_bounds__(kMetricThreads) void k_usage_part(int32_t* usage, int64_t N, UsagePart* parts,
                                                               int reset) {
    __shared__ double sh_cl[kMetricThreads];
    __shared__ unsigned long long sh_tot[kMetricThreads], sh_nz[kMetricThreads], sh_comp[kMetricThreads];
    const int b = blockIdx.y, part = blockIdx.x, tid = threadIdx.x;
    const int64_t span = (N + kUsageParts - 1) / kUsageParts;
    const int64_t lo = part * span, hi = min(N, lo + span);
    int32_t* u = usage + static_cast<size_t>(b) * N;
    unsigned long long tot = 0, nz = 0, comp = 0;
    double cl = 0.0;
    for (int64_t i = lo + tid; i < hi; i += kMetricThreads) {
        const int32_t c = u[i];
        if (c > 0) {
            tot += static_cast<unsigned long long>(c);
            nz += 1;
            if (c > 1) {
                comp += static_cast<unsigned long long>(c);
                const double cd = static_cast<double>(c);
                cl += cd * log(cd);
            }
        }
        if (reset && c != 0) u[i] = 0;
    }
    sh_cl[tid] = cl; sh_tot[tid] = tot; sh_nz[tid] = nz; sh_comp[tid] = comp;
    __syncthreads();
    for (int st = kMetricThreads / 2; st > 0; st >>= 1) {
        if (tid < st) {
            sh_cl[tid] += sh_cl[tid + st];
            sh_tot[tid] += sh_tot[tid + st];
            sh_nz[tid] += sh_nz[tid + st];
            sh_comp[tid] += sh_comp[tid + st];
        }
        __syncthreads();
    }
    if (tid == 0) parts[static_cast<size_t>(b) * kUsageParts + part] = UsagePart{sh_cl[0], sh_tot[0], sh_nz[0], sh_comp[0]};
}

// The slices of sequence b added in slice order, then the metrics.
__global__ void k_usage_final(const UsagePart* parts, int B, int64_t N, double* metrics) {
    const int b = blockIdx.x * blockDim.x + threadIdx.x;
    if (b >= B) return;
    double cl = 0.0;
    unsigned long long tot = 0, nz = 0, comp = 0;
    for (int i = 0; i < kUsageParts; ++i) {
        const UsagePart& q = parts[static_cast<size_t>(b) * kUsageParts + i];
        cl += q.cl; tot += q.tot; nz += q.nz; comp += q.comp;
    }
    double* m = metrics + static_cast<size_t>(b) * 4;
    const double S = static_cast<double>(tot), Nd = static_cast<double>(N);
    m[0] = static_cast<double>(nz) / Nd;
    m[1] = S > 0.0 ? static_cast<double>(comp) / S : 0.0;
    m[2] = S > 0.0 ? cl / S + log(Nd) - log(S) : 0.0;
    m[3] = S;
}

}  // namespace

hipError_t launch_usage_metrics(int32_t* usage, int B, int64_t N, void* scratch, double* metrics, int reset,
                                hipStream_t s) {
    if (B <= 0) return hipSuccess;
    auto* parts = static_cast<UsagePart*>(scratch);
    hipLaunchKernelGGL(k_usage_part, dim3(kUsageParts, static_cast<unsigned>(B)), dim3(kMetricThreads), 0, s, usage,
                       N, parts, reset);
    hipLaunchKernelGGL(k_usage_final, dim3(static_cast<unsigned>((B + 63) / 64)), dim3(64), 0, s, parts, B, N,
                       metrics);
    return hipGetLastError();
}

}  // namespace fwpkm
