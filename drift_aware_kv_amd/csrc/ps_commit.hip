// Polestar-Commit on the drift this library measures (technical summary
// section 2.B): the current-block rule, a drift delta against a
// confidence-conditioned threshold, and the suffix-block rule, driven by the
// top-k drifted clusters.
//
// Both kernels are tiny and bound by launch latency: one workgroup per window,
// a few KiB of reads.  The current-block rule does its arithmetic in fp64,
// one IEEE operation at a time, so its decision is reproducible bit for bit.
#include "ps_common.h"

namespace {

using namespace ps;

// One workgroup per window.  Every thread reads the window's history count
// before thread 0 advances it (barrier between the read and the write).
__global__ __launch_bounds__(64) void k_commit_block(const float* __restrict__ D_i,
                                                     const float* __restrict__ conf, int N, int Nb,
                                                     int block_start, float alpha, float tau_s,
                                                     double* __restrict__ hist_sum,
                                                     int32_t* __restrict__ hist_n,
                                                     uint8_t* __restrict__ commit,
                                                     float* __restrict__ delta)
{
    const int w = blockIdx.x;
    const int32_t n0 = hist_n[w];
    const int32_t n = n0 > 0 ? n0 : 0;
    for (int i = threadIdx.x; i < Nb; i += blockDim.x) {
        const size_t r = (size_t)w * Nb + i;
        const double D = (double)D_i[r];
        const float c = conf[(size_t)w * N + block_start + i];
        double prev = 0.0, dl = 0.0;
        int drift_rule = 0;
        if (n > 0) {
            prev = hist_sum[r];
            const double mean = prev / (double)n;
            const double gap = (double)tau_s - (double)c;
            dl = D - mean;
            drift_rule = dl > (double)alpha * (gap * gap);
        }
        const int conf_rule = c >= tau_s;
        commit[r] = (uint8_t)(drift_rule | (conf_rule << 1));
        if (delta) delta[r] = (float)dl;
        hist_sum[r] = prev + D;
    }
    __syncthreads();
    if (threadIdx.x == 0) hist_n[w] = n + 1;
}

// One workgroup per window: member and suffix-member counts of every cluster
// in LDS (integer atomics, so the counts are exact), then the top-k test and
// the confidence mask.
__global__ __launch_bounds__(1024) void k_commit_suffix(const int32_t* __restrict__ assign,
                                                       const int32_t* __restrict__ idx, int k, int N,
                                                       int K, int first,
                                                       const float* __restrict__ conf, float tau_s,
                                                       uint8_t* __restrict__ flag,
                                                       uint8_t* __restrict__ commit)
{
    __shared__ int members[kMaxK];
    __shared__ int in_suffix[kMaxK];
    const int w = blockIdx.x, t = threadIdx.x;
    for (int c = t; c < K; c += blockDim.x) {
        members[c] = 0;
        in_suffix[c] = 0;
    }
    __syncthreads();
    const int32_t* a = assign + (size_t)w * N;
    for (int j = t; j < N; j += blockDim.x) {
        const int c = a[j];
        if ((unsigned)c < (unsigned)K) {
            atomicAdd(&members[c], 1);
            if (j >= first) atomicAdd(&in_suffix[c], 1);
        }
    }
    __syncthreads();
    int f = 0;
    for (int r = t; r < k; r += blockDim.x) {
        const int c = idx[(size_t)w * k + r];
        if ((unsigned)c < (unsigned)K && 2 * in_suffix[c] > members[c]) f = 1;
    }
    f = __syncthreads_or(f);
    if (t == 0) flag[w] = (uint8_t)f;
    const float* cw = conf + (size_t)w * N;
    uint8_t* out = commit + (size_t)w * N;
    for (int j = t; j < N; j += blockDim.x) out[j] = (uint8_t)(f && j >= first && cw[j] >= tau_s);
}

ps_status check_rows(const ps_shape* s, int32_t block_start)
{
    if (s->W < 0 || s->N < 1 || s->N >= (1 << 24) || s->Nb < 0 || s->Nb > s->N) return PS_ERR_SHAPE;
    if (block_start < 0 || block_start > s->N - s->Nb) return PS_ERR_RANGE;
    return PS_OK;
}

}  // namespace

extern "C" ps_status ps_commit_block(const ps_shape* s, const float* D_i, const float* conf,
                                     int32_t block_start, float alpha, float tau_s,
                                     double* hist_sum, int32_t* hist_n, uint8_t* commit,
                                     float* delta, void* stream)
{
    using namespace ps_host;
    if (!s || !D_i || !conf || !hist_sum || !hist_n || !commit) return PS_ERR_NULL;
    ps_status st = check_rows(s, block_start);
    if (st != PS_OK) return st;
    if (!std::isfinite(alpha) || alpha < 0.0f || !std::isfinite(tau_s)) return PS_ERR_RANGE;
    if (!aligned16(D_i) || !aligned16(conf) || !aligned16(hist_sum) || !aligned16(hist_n) ||
        !aligned16(commit) || (delta && !aligned16(delta)))
        return PS_ERR_ALIGN;
    if (s->W == 0) return PS_OK;
    hipStream_t stm = (hipStream_t)stream;
    (void)hipGetLastError();
    PS_LAUNCH("k_commit_block", k_commit_block, dim3(s->W), dim3(64), 0, stm, D_i, conf, s->N,
              s->Nb, block_start, alpha, tau_s, hist_sum, hist_n, commit, delta);
    return hipGetLastError() == hipSuccess ? PS_OK : PS_ERR_DEVICE;
}

extern "C" ps_status ps_commit_suffix(const ps_shape* s, const int32_t* assign, const int32_t* idx,
                                      int32_t k, int32_t block_start, const float* conf,
                                      float tau_s, uint8_t* flag, uint8_t* commit, void* stream)
{
    using namespace ps_host;
    if (!s || !assign || !idx || !conf || !flag || !commit) return PS_ERR_NULL;
    ps_status st = check_rows(s, block_start);
    if (st != PS_OK) return st;
    if (s->K < 1 || s->K > kMaxK) return PS_ERR_SHAPE;
    if (k < 1 || k > s->K || !std::isfinite(tau_s)) return PS_ERR_RANGE;
    if (!aligned16(assign) || !aligned16(idx) || !aligned16(conf) || !aligned16(flag) ||
        !aligned16(commit))
        return PS_ERR_ALIGN;
    if (s->W == 0) return PS_OK;
    hipStream_t stm = (hipStream_t)stream;
    (void)hipGetLastError();
    PS_LAUNCH("k_commit_suffix", k_commit_suffix, dim3(s->W), dim3(1024), 0, stm, assign, idx, k,
              s->N, s->K, block_start + s->Nb, conf, tau_s, flag, commit);
    return hipGetLastError() == hipSuccess ? PS_OK : PS_ERR_DEVICE;
}
