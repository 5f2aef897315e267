// budget_schedule.hip -- confidence-driven verify budgets for MI355X (gfx950).
//
// What is computed: "Speculative decoding becomes standard: DSpark and
// multi-token drafters", section "What DSpark adds", paragraph 2 (each
// drafted position has a confidence, read as its chance of acceptance once
// every earlier position of the block was accepted; the verify window of
// every request is sized jointly across the batch for accepted tokens per
// unit of verification, and shrinks as load grows), and the Analytics
// Vidhya DSpark page, section
// "Gotchas and Issues" (a cutoff recomputed for every batch; verify only
// what has positive expected value). Reading: verifying position k of
// request b adds g[b, k] = prod_{l <= k} c[b, l] expected accepted tokens;
// the batch verifies the N largest gains above tau, equal gains taken by
// position, then request; k_b is the number of positions taken from b (a
// prefix, since gains never increase along a block).
//
// Design: one workgroup of 1024 threads; thread t owns a contiguous range of
// at most 16 requests. Their gains (left-to-right fp32 products: the same
// bits as any other implementation that multiplies in that order) are kept
// in LDS when the batch's B*K gains fit, else recomputed from the
// confidences on every pass. The N-th largest gain is found by a 4-pass,
// 8-bit radix select over the gains' bit patterns (monotone for non-negative
// floats) with an LDS histogram; equal gains at the cut are resolved with
// per-position counts and one block scan over requests. No workspace and no
// global atomics.

#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdint>

#include "spec_verify.h"

namespace {

constexpr int kSchedThreads = 1024;
constexpr int kSchedWaves = kSchedThreads / 64;
constexpr int kLdsGains = 12288;        // B*K up to this: gains kept in LDS (48 KB)

// Confidence as the scheduler reads it: NaN and negatives are 0, values
// above 1 are 1, and -0 becomes +0 (so every gain is a non-negative float
// whose bit pattern orders like its value).
__device__ __forceinline__ float clamp_conf(float c) {
    return c >= 0.0f ? fminf(c, 1.0f) + 0.0f : 0.0f;
}

struct SchedShared {
    unsigned hist[2][256];          // radix histograms, alternating by pass
    unsigned level[SV_MAX_K + 1];
    unsigned wsum[kSchedWaves];
    unsigned total;
    unsigned digit, above;          // radix step: chosen digit, keys in higher bins
    int cut_level, cut_rank;        // ties: the partial level and how many it takes
};

// Exclusive prefix over threads in thread order (each thread one count).
__device__ unsigned block_exclusive(SchedShared& sh, unsigned v) {
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    unsigned incl = v;
    #pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
        const unsigned u = __shfl_up(incl, o, 64);
        if (lane >= o) incl += u;
    }
    if (lane == 63) sh.wsum[wave] = incl;
    __syncthreads();
    unsigned base = 0;
    for (int w = 0; w < wave; ++w) base += sh.wsum[w];
    __syncthreads();
    return base + incl - v;
}

template <bool kLds>
__global__ __launch_bounds__(kSchedThreads) void budget_schedule_kernel(
    const float* __restrict__ conf, int B, int K, int n_total, float tau,
    int32_t* __restrict__ out) {
    __shared__ SchedShared sh;
    extern __shared__ float gl[];          // kLds: gains [B * K]
    const int tid = threadIdx.x;
    const int per = (B + kSchedThreads - 1) / kSchedThreads;
    const int b0 = min(tid * per, B), b1 = min(b0 + per, B);

    if (kLds) {
        for (int b = b0; b < b1; ++b) {
            const float* row = conf + (size_t)b * K;
            float run = 1.0f;
            for (int k = 0; k < K; ++k) {
                run = run * clamp_conf(row[k]);
                gl[b * K + k] = run;
            }
        }
        // Each thread reads only its own requests' gains: no barrier needed.
    }

    // Calls f(k, gain) for every position of request b, in position order.
    auto row_gains = [&](int b, auto&& f) {
        if (kLds) {
            for (int k = 0; k < K; ++k) f(k, gl[b * K + k]);
        } else {
            const float* row = conf + (size_t)b * K;
            float run = 1.0f;
            for (int k = 0; k < K; ++k) {
                run = run * clamp_conf(row[k]);
                f(k, run);
            }
        }
    };
    // The same over all of this thread's requests, in request order.
    auto each_gain = [&](auto&& f) {
        for (int b = b0; b < b1; ++b) row_gains(b, [&](int k, float g) { f(b, k, g); });
    };

    // Radix select of the N-th largest candidate key (candidates: gains
    // above tau; key: the gain's bit pattern), 8 bits per pass from the top.
    // A request's gains never increase along its block, so the keys that
    // match the current prefix are one run of positions whose digits never
    // increase: each thread adds run lengths, a few atomics per request. The
    // first pass's histogram also counts the candidates; with no more of
    // them than N (or N == 0) no cut is needed.
    if (tid < 512) (&sh.hist[0][0])[tid] = 0;
    if (tid <= SV_MAX_K) sh.level[tid] = 0;
    __syncthreads();
    bool all = true;
    unsigned cut = 0, need = 0;
    unsigned prefix = 0, mask = 0, remaining = (unsigned)n_total;
    for (int pass = 0; pass < 4; ++pass) {
        const int shift = 24 - 8 * pass;
        unsigned* h = sh.hist[pass & 1];
        for (int b = b0; b < b1; ++b) {
            int run_bin = -1;
            unsigned run_len = 0;
            row_gains(b, [&](int, float g) {
                const unsigned key = __float_as_uint(g);
                const int bin = (g > tau && (key & mask) == prefix) ? (int)((key >> shift) & 255u) : -1;
                if (bin != run_bin) {
                    if (run_bin >= 0) atomicAdd(&h[run_bin], run_len);
                    run_bin = bin;
                    run_len = 0;
                }
                if (bin >= 0) ++run_len;
            });
            if (run_bin >= 0) atomicAdd(&h[run_bin], run_len);
        }
        // The other histogram was last read before the previous pass's
        // second barrier: clear it for the next pass.
        if (tid < 256) sh.hist[(pass + 1) & 1][tid] = 0;
        __syncthreads();
        if (tid < 64) {
            // Lane l holds bins 4l .. 4l+3; suffix sums from the top bin.
            unsigned c[4], sl = 0;
            #pragma unroll
            for (int q = 0; q < 4; ++q) {
                c[q] = h[4 * tid + q];
                sl += c[q];
            }
            unsigned suf = sl;                 // bins 4l .. 255
            #pragma unroll
            for (int o = 1; o < 64; o <<= 1) {
                const unsigned u = __shfl_down(suf, o, 64);
                if (tid + o < 64) suf += u;
            }
            if (tid == 0) sh.total = suf;      // keys counted in this pass
            const unsigned higher = suf - sl;  // bins above this lane's four
            // The lane whose bins hold the remaining-th largest key.
            if (higher < remaining && suf >= remaining) {
                unsigned acc = higher;
                int d = 4 * tid + 3;
                for (int q = 3; q >= 0; --q) {
                    if (acc + c[q] >= remaining) {
                        d = 4 * tid + q;
                        break;
                    }
                    acc += c[q];
                }
                sh.digit = (unsigned)d;
                sh.above = acc;
            }
        }
        __syncthreads();
        if (pass == 0) {
            all = n_total == 0 || (unsigned)n_total >= sh.total;
            if (all) break;
        }
        remaining -= sh.above;
        prefix |= sh.digit << shift;
        mask |= 255u << shift;
    }
    if (!all) {
        cut = prefix;
        need = remaining;
    }

    // Per request: s_b = positions above the cut, e_b = positions at or above
    // it (gains never increase along a block, so both are prefixes and the
    // positions equal to the cut are [s_b, e_b)).
    auto above_cut = [&](float g) -> bool {
        return all ? (n_total > 0 && g > tau) : (g > tau && __float_as_uint(g) > cut);
    };
    auto at_cut = [&](float g) -> bool {
        return !all && g > tau && __float_as_uint(g) == cut;
    };
    if (need > 0) {
        each_gain([&](int, int k, float g) {
            if (at_cut(g)) atomicAdd(&sh.level[k], 1u);
        });
    }
    __syncthreads();
    if (tid == 0) {
        // Levels (positions) in order: full levels, then a partial one.
        int lv = K;
        unsigned acc = 0;
        for (int k = 0; k < K && need > 0; ++k) {
            if (acc + sh.level[k] >= need) {
                lv = k;
                break;
            }
            acc += sh.level[k];
        }
        sh.cut_level = lv;
        sh.cut_rank = (int)(need - acc);
    }
    __syncthreads();
    const int lv = sh.cut_level;
    const unsigned rank_need = need > 0 ? (unsigned)sh.cut_rank : 0u;

    // Which of this thread's requests have the partial level among their
    // equal positions, then their rank among all such requests (b order).
    unsigned on_level = 0;
    if (need > 0) {
        each_gain([&](int, int k, float g) {
            if (k == lv && at_cut(g)) ++on_level;
        });
    }
    unsigned rank = block_exclusive(sh, on_level);
    for (int b = b0; b < b1; ++b) {
        int s = 0, e = 0;
        bool lv_here = false;
        auto visit = [&](int k, float g) {
            if (above_cut(g)) ++s;
            if (above_cut(g) || at_cut(g)) ++e;
            if (k == lv && at_cut(g)) lv_here = true;
        };
        row_gains(b, visit);
        int kb = s + max(0, min(e, lv) - s);
        if (lv_here) {
            if (rank < rank_need) ++kb;
            ++rank;
        }
        out[b] = kb;
    }
}

bool aligned4(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 3u) == 0; }

}  // namespace

extern "C" int spec_budget_schedule(const float* confidences, int B, int K, int n_total,
                                    float tau, int32_t* out_budgets, void* stream) {
    if (B < 0 || B > SV_MAX_BATCH || K < 0 || K > SV_MAX_K || n_total < 0 ||
        !std::isfinite(tau) || tau < 0.0f) {
        return SV_ERR_ARG;
    }
    if (B == 0) return SV_OK;
    if (!out_budgets || (K > 0 && !confidences)) return SV_ERR_NULL;
    if (!aligned4(out_budgets) || (K > 0 && !aligned4(confidences))) return SV_ERR_ALIGN;
    const hipStream_t s = static_cast<hipStream_t>(stream);
    if ((long long)B * K <= kLdsGains) {
        hipLaunchKernelGGL(budget_schedule_kernel<true>, dim3(1), dim3(kSchedThreads),
                           (size_t)B * K * sizeof(float), s, confidences, B, K, n_total, tau,
                           out_budgets);
    } else {
        hipLaunchKernelGGL(budget_schedule_kernel<false>, dim3(1), dim3(kSchedThreads), 0, s,
                           confidences, B, K, n_total, tau, out_budgets);
    }
    return hipGetLastError() == hipSuccess ? SV_OK : SV_ERR_HIP;
}
