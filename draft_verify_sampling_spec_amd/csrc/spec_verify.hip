// spec_verify.hip -- batched draft verification for MI355X (gfx950, wave64).
//
// What is computed: "Speculative decoding becomes standard: DSpark and
// multi-token drafters", section "Why draft-and-verify does not change the
// output" (greedy keep-while-agreeing rule, paragraph 1; the sampled
// min(1, p/q) acceptance with residual resampling, paragraph 2), with the
// per-request verify budgets of section "What DSpark adds", paragraph 2.
// The ABI and its conventions are documented in include/spec_verify.h.
//
// Design: one persistent kernel per call, every logit byte read from HBM once.
//  * Work unit = vocabulary chunk c of position i of request b: the chunk of
//    target row i and, for a drafted position, the same chunk of drafter row
//    i. Every chunk has the same size (448 data lanes x 4 sixteen-byte loads
//    per row). Units are numbered request-major, position-major, chunk-minor,
//    so the C chunks of one position (a "team") are consecutive.
//  * The grid is exactly the resident workgroups; workgroup w takes units
//    w, w + G, w + 2G, ... (G = grid size >= C, so two units of one
//    workgroup never share a team).
//  * A workgroup is 8 waves. Waves 1-7 stream data: 16-byte loads of a unit
//    into registers, all in flight at once, reduced to the chunk's max and
//    sum of 2^((z - max) log2(e)/T) (sampled) or (max, lowest index)
//    (greedy). Wave 0 is the control wave: it publishes the partials with
//    device-scope stores, counts the team's arrivals (the last arriver leads
//    the team: merges the chunks, takes the accept decision, publishes the
//    normalisers) and waits on other teams, so that no data wave ever waits
//    on a synchronisation load behind its own prefetched loads.
//  * The unit's data then waits in a per-lane LDS slot while the workgroup
//    streams its next unit; then the control wave reads the parked team's
//    decision. Only for the request's earliest rejected position do the
//    members turn the parked chunk into its residual mass max(0, p - q); the
//    last of them scans the residual CDF over chunks, and the data waves
//    re-read just the one chunk holding the threshold for the element-level
//    scan. The bonus draw works the same way on the target row alone.
//  * Per request, the team that completes last writes the outputs.
//  * Waiting: a workgroup waits for a team only after arriving at it, and
//    while it holds just the unit after it, which lies G >= C units further
//    on; by induction on the unit index every unit arrives. The wait is
//    still bounded (status flag on expiry) so the kernel always drains.
//  * Synchronisation uses device-scope relaxed atomics plus s_waitcnt, never
//    release/acquire fences (those write back and invalidate the whole L2).
//  * Counters clean themselves: each is zeroed by its last user.

#include <hip/hip_runtime.h>

#include <climits>
#include <cmath>
#include <cstdint>
#include <cstring>
#include <type_traits>

#include "spec_verify.h"

namespace {

// The wave count is a multiple of 4 so that every SIMD of a CU holds the same
// number of waves of each workgroup: with 5 waves, the hardware reserves two
// wave slots per SIMD for each workgroup, and fewer workgroups fit than the
// occupancy query reports.
constexpr int kWaves = 8;                      // wave 0: control; waves 1-7: data
constexpr int kThreads = kWaves * 64;
constexpr int kDataWaves = kWaves - 1;
constexpr int kDataThreads = kDataWaves * 64;
constexpr int kG = 4;                          // 16-byte groups per data lane per row of a unit
constexpr int kScanElems = kDataThreads * 8;   // elements per scan sub-tile
constexpr int kMaxSub = 4;                     // sub-tiles per chunk (chunk <= 8192 elements)
constexpr int kTeamWords = 32;                 // words per team record (128 bytes)
constexpr int kReqStride = 16;                 // words between request records (64 bytes)
constexpr unsigned kNoReject = 0x7F7F7F7Fu;    // "no rejection yet" (memset pattern)
constexpr unsigned kSpinLimit = 1u << 20;      // bounded wait, about 0.1 s

// Team record words.
constexpr int TW_ARRIVE = 0;    // units of the team that published their partials
constexpr int TW_PHASE = 1;     // (call epoch << 2) | PH_* bits once the leader has published
constexpr int TW_ST = 2;        // double S_t (words 2-3)
constexpr int TW_SD = 4;        // double S_d (words 4-5)
constexpr int TW_MT = 6;        // float M_t
constexpr int TW_MD = 7;        // float M_d
constexpr int TW_ARRIVE2 = 8;   // units that published their residual mass
constexpr unsigned PH_READY = 1u;
constexpr unsigned PH_RESIDUAL = 2u;

// Partial record of one unit (four 64-bit words):
//   [0] sampled: (M_t bits << 32) | M_d bits    greedy: (max bits << 32) | index
//   [1] S_t = sum over the chunk of 2^((z_t - M_t) c)   (double)
//   [2] S_d (double)
//   [3] residual mass of the chunk once the normalisers are known (double)
constexpr int kPartWords = 4;

// Philox4x32 constants (Salmon et al., SC'11): round multipliers and the key
// increments applied between rounds.
constexpr uint32_t kPhiloxM0 = 0xD2511F53u;
constexpr uint32_t kPhiloxM1 = 0xCD9E8D57u;
constexpr uint32_t kPhiloxW0 = 0x9E3779B9u;
constexpr uint32_t kPhiloxW1 = 0xBB67AE85u;

constexpr double kLog2e = 1.4426950408889634073599246810019;

struct Params {
    const void* target;            // [B, K+1, V]
    const void* draft;             // [B, K, V] (sampled mode)
    const int32_t* tokens;         // [B, K]
    const int32_t* budgets;        // [B]
    int32_t* out_tokens;           // [B, K+1]
    int32_t* out_nacc;             // [B]
    float* out_p;                  // [B, K] or null
    float* out_q;                  // [B, K] or null
    unsigned long long* part;      // [B*(K+1)*C][kPartWords]
    unsigned* team;                // [B*(K+1)][kTeamWords]
    unsigned long long* result;    // [B*(K+1)]: (accepted << 32) | drawn token
    unsigned* req_count;           // [B][kReqStride]: teams completed
    unsigned* req_first;           // [B][kReqStride]: first rejected position
    unsigned* status;              // 1 word
    int B, K, V;
    int C;                         // chunks per row
    int CE;                        // elements per chunk
    float c32;                     // log2(e) / T
    double c64;
    uint32_t key0, key1;
    unsigned epoch;                // call number (30 bits, never 0): tags phase words
};

// ------------------------------------------------------------- atomics --

__device__ __forceinline__ void st32(unsigned* p, unsigned v) {
    __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ unsigned ld32(unsigned* p) {
    return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void st64(unsigned long long* p, unsigned long long v) {
    __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ unsigned long long ld64(unsigned long long* p) {
    return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ unsigned add32(unsigned* p, unsigned v) {
    return __hip_atomic_fetch_add(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
// Wait until every memory operation this wave issued has completed, so that
// device-scope stores above are visible before the counter update below.
// The signal fences only stop the compiler from moving memory operations
// across the wait; they emit no instruction.
__device__ __forceinline__ void drain() {
    __atomic_signal_fence(__ATOMIC_SEQ_CST);
    __builtin_amdgcn_s_waitcnt(0);
    __atomic_signal_fence(__ATOMIC_SEQ_CST);
}

__device__ __forceinline__ unsigned long long as_u64(double d) {
    return (unsigned long long)__double_as_longlong(d);
}
__device__ __forceinline__ double as_f64(unsigned long long u) {
    return __longlong_as_double((long long)u);
}

// ----------------------------------------------------------------- Philox --

__device__ __forceinline__ uint4 philox4x32_10(uint32_t c0, uint32_t c1, uint32_t c2,
                                               uint32_t c3, uint32_t k0, uint32_t k1) {
    #pragma unroll
    for (int r = 0; r < 10; ++r) {
        if (r > 0) {
            k0 += kPhiloxW0;
            k1 += kPhiloxW1;
        }
        const uint32_t lo0 = kPhiloxM0 * c0, hi0 = __umulhi(kPhiloxM0, c0);
        const uint32_t lo1 = kPhiloxM1 * c2, hi1 = __umulhi(kPhiloxM1, c2);
        const uint32_t n0 = hi1 ^ c1 ^ k0;
        const uint32_t n2 = hi0 ^ c3 ^ k1;
        c0 = n0;
        c1 = lo1;
        c2 = n2;
        c3 = lo0;
    }
    return make_uint4(c0, c1, c2, c3);
}

__device__ __forceinline__ double word_to_uniform(uint32_t w) {
    return (double)(w >> 8) * (1.0 / 16777216.0);
}

// ---------------------------------------------------------- element types --

// A "group" is the 16 bytes one lane loads at once: 8 bf16 or 4 fp32 values.
template <typename E> struct Elem;

template <> struct Elem<float> {
    static constexpr int W = 4;
    static constexpr uint32_t kNegInfWord = 0xFF800000u;
    __device__ static __forceinline__ float at(const uint4& g, int k) {
        const uint32_t w = k == 0 ? g.x : k == 1 ? g.y : k == 2 ? g.z : g.w;
        return __uint_as_float(w);
    }
    __device__ static __forceinline__ float one(const float* p) { return *p; }
    __device__ static __forceinline__ void put(uint32_t* w, int k, const float* p) {
        w[k] = __float_as_uint(*p);
    }
};

template <> struct Elem<uint16_t> {   // bfloat16 bit patterns
    static constexpr int W = 8;
    static constexpr uint32_t kNegInfWord = 0xFF80FF80u;
    __device__ static __forceinline__ float at(const uint4& g, int k) {
        const uint32_t w = (k >> 1) == 0 ? g.x : (k >> 1) == 1 ? g.y : (k >> 1) == 2 ? g.z : g.w;
        return (k & 1) ? __uint_as_float(w & 0xFFFF0000u) : __uint_as_float(w << 16);
    }
    __device__ static __forceinline__ float one(const uint16_t* p) {
        return __uint_as_float((uint32_t)(*p) << 16);
    }
    __device__ static __forceinline__ void put(uint32_t* w, int k, const uint16_t* p) {
        const uint32_t sh = (k & 1) * 16;
        w[k >> 1] = (w[k >> 1] & ~(0xFFFFu << sh)) | ((uint32_t)(*p) << sh);
    }
};

template <typename E>
__device__ __forceinline__ uint4 neg_group() {
    return make_uint4(Elem<E>::kNegInfWord, Elem<E>::kNegInfWord, Elem<E>::kNegInfWord,
                      Elem<E>::kNegInfWord);
}

// Load the group of elements [e, e + W) of a row segment of n elements;
// elements at or beyond n read as -inf. `vec_ok`: 16-byte loads are legal.
template <typename E, bool kVec = false>
__device__ __forceinline__ uint4 load_group(const E* base, int e, int n, bool vec_ok) {
    constexpr int W = Elem<E>::W;
    if (kVec) {
        // Caller guarantees 16-byte alignment and that n is a multiple of W.
        return e < n ? *reinterpret_cast<const uint4*>(base + e) : neg_group<E>();
    }
    if (vec_ok && e + W <= n) {
        return *reinterpret_cast<const uint4*>(base + e);
    }
    uint32_t w[4] = {Elem<E>::kNegInfWord, Elem<E>::kNegInfWord, Elem<E>::kNegInfWord,
                     Elem<E>::kNegInfWord};
    #pragma unroll
    for (int k = 0; k < W; ++k) {
        if (e + k < n) Elem<E>::put(w, k, base + e + k);
    }
    return make_uint4(w[0], w[1], w[2], w[3]);
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

__device__ __forceinline__ bool aligned16(const void* p) {
    return (reinterpret_cast<uintptr_t>(p) & 15) == 0;
}

// --------------------------------------------------------- shared memory --

struct Shared {
    float red_m[kWaves][2];          // block max of (target, drafter)
    double red_s[kWaves][2];         // block sums
    float red_f[kWaves];
    int red_i[kWaves];
    double red_d[kWaves];
    double scan_ws[kMaxSub * kDataWaves];
    int leader;
    int leader2;
    unsigned phase;
    float nmt, nmd;                  // normalisers of the team being finished
    double nst, nsd;
    // chunk scan hand-off (control wave -> data waves)
    int scan_chunk;
    int scan_residual;               // 1: residual p - q; 0: target row alone
    double scan_thr;                 // threshold relative to the chunk start
    int sub_star;
    double sub_base;
    // deferred draws, run by the data waves at the start of the next round
    int pend_bonus;
    int bonus_b, bonus_k, bonus_tr, bonus_chunk;
    float bonus_mt, bonus_ist;
    double bonus_thr;
    int pend_resid;
    int resid_b, resid_i, resid_k, resid_tr;
    float resid_mt, resid_md, resid_ist, resid_isd;
};

// ------------------------------------------------------ block reductions --

__device__ __forceinline__ float wave_max(float v) {
    #pragma unroll
    for (int off = 32; off > 0; off >>= 1) v = fmaxf(v, __shfl_xor(v, off, 64));
    return v;
}

__device__ __forceinline__ double wave_sum(double v) {
    #pragma unroll
    for (int off = 32; off > 0; off >>= 1) v += __shfl_xor(v, off, 64);
    return v;
}

// Inclusive prefix sum over the 64 lanes of a wave, in lane order.
__device__ __forceinline__ double wave_incl_scan(double v, int lane) {
    #pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
        const double o = __shfl_up(v, off, 64);
        if (lane >= off) v += o;
    }
    return v;
}

__device__ __forceinline__ bool better_arg(float v, int i, float bv, int bi) {
    return v > bv || (v == bv && i < bi);
}

// Block-wide max of two values (every thread gets both results). The control
// wave contributes -inf.
__device__ __forceinline__ float2 block_max2(Shared& sh, float a, float b) {
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    a = wave_max(a);
    b = wave_max(b);
    if (lane == 0) {
        sh.red_m[wave][0] = a;
        sh.red_m[wave][1] = b;
    }
    __syncthreads();
    float ra = sh.red_m[0][0], rb = sh.red_m[0][1];
    #pragma unroll
    for (int w = 1; w < kWaves; ++w) {
        ra = fmaxf(ra, sh.red_m[w][0]);
        rb = fmaxf(rb, sh.red_m[w][1]);
    }
    return make_float2(ra, rb);
}

// Block-wide sums of two doubles (every thread gets both results). Callers
// separate consecutive uses by at least one other barrier.
__device__ __forceinline__ double2 block_sum2(Shared& sh, double a, double b) {
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    a = wave_sum(a);
    b = wave_sum(b);
    if (lane == 0) {
        sh.red_s[wave][0] = a;
        sh.red_s[wave][1] = b;
    }
    __syncthreads();
    double ra = sh.red_s[0][0], rb = sh.red_s[0][1];
    #pragma unroll
    for (int w = 1; w < kWaves; ++w) {
        ra += sh.red_s[w][0];
        rb += sh.red_s[w][1];
    }
    return make_double2(ra, rb);
}

// ------------------------------------------------------- mass and scans --

// Sampling mass of the 8 elements [e, e + 8) of a chunk of n elements:
// residual max(0, p - q) when rd is given, else p. p = 2^((z_t - mt) c) / S_t.
template <typename E, bool kVec>
__device__ __forceinline__ void mass8(const E* rt, const E* rd, int e, int n, bool vt, bool vd,
                                      float mt, float ist, float md, float isd, float c,
                                      float r[8]) {
    constexpr int W = Elem<E>::W;
    #pragma unroll
    for (int h = 0; h < 8 / W; ++h) {
        const uint4 gt = load_group<E, kVec>(rt, e + h * W, n, vt);
        if (rd != nullptr) {
            const uint4 gd = load_group<E, kVec>(rd, e + h * W, n, vd);
            #pragma unroll
            for (int k = 0; k < W; ++k) {
                const float p = fast_exp2((Elem<E>::at(gt, k) - mt) * c) * ist;
                const float q = fast_exp2((Elem<E>::at(gd, k) - md) * c) * isd;
                r[h * W + k] = fmaxf(0.0f, p - q);
            }
        } else {
            #pragma unroll
            for (int k = 0; k < W; ++k) r[h * W + k] = fast_exp2((Elem<E>::at(gt, k) - mt) * c) * ist;
        }
    }
}

// Element-level inverse CDF inside one chunk (whole workgroup; the data
// waves hold the elements): returns the offset in the chunk of the smallest
// element whose running mass (from the chunk start) exceeds thr, zero-mass
// elements excluded; if rounding leaves no crossing, the last positive-mass
// element; -1 if the chunk has no mass.
template <typename E, bool kVec>
__device__ int chunk_scan(Shared& sh, const E* rt, const E* rd, int n, float mt, float ist,
                          float md, float isd, float c, double thr) {
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const bool data = wave > 0;
    const int dt = tid - 64;                       // data thread index
    const bool vt = aligned16(rt);
    const bool vd = rd != nullptr && aligned16(rd);
    const int nsub = (n + kScanElems - 1) / kScanElems;
    for (int s = 0; s < nsub; ++s) {
        float ls = 0.0f;
        if (data) {
            float r[8];
            mass8<E, kVec>(rt, rd, s * kScanElems + dt * 8, n, vt, vd, mt, ist, md, isd, c, r);
            #pragma unroll
            for (int k = 0; k < 8; ++k) ls += r[k];
        }
        const double ws = wave_sum((double)ls);
        if (data && lane == 0) sh.scan_ws[s * kDataWaves + wave - 1] = ws;
    }
    __syncthreads();
    if (tid == 0) {
        double acc = 0.0, acc_last = 0.0;
        int star = -1, last = -1;
        for (int s = 0; s < nsub; ++s) {
            const double* ws = sh.scan_ws + s * kDataWaves;
            double tot = ws[0];
            for (int w = 1; w < kDataWaves; ++w) tot += ws[w];
            if (tot > 0.0) {
                last = s;
                acc_last = acc;
                if (acc + tot > thr) {
                    star = s;
                    break;
                }
            }
            acc += tot;
        }
        if (star < 0) {
            star = last;
            acc = acc_last;
        }
        sh.sub_star = star;
        sh.sub_base = acc;
    }
    __syncthreads();
    const int s = sh.sub_star;
    if (s < 0) {
        __syncthreads();
        return -1;
    }
    const int e = s * kScanElems + dt * 8;
    float r[8];
    #pragma unroll
    for (int k = 0; k < 8; ++k) r[k] = 0.0f;
    if (data) mass8<E, kVec>(rt, rd, e, n, vt, vd, mt, ist, md, isd, c, r);
    double pre[8];
    double run = 0.0;
    #pragma unroll
    for (int k = 0; k < 8; ++k) {
        run += (double)r[k];
        pre[k] = run;
    }
    const double incl = wave_incl_scan(run, lane);
    if (lane == 63) sh.red_d[wave] = incl;
    __syncthreads();
    const double up = __shfl_up(incl, 1, 64);
    double excl = lane ? up : 0.0;
    for (int w = 1; w < wave; ++w) excl += sh.red_d[w];
    const double t = thr - sh.sub_base;
    int cand = INT_MAX, last_pos = -1;
    if (data) {
        #pragma unroll
        for (int k = 0; k < 8; ++k) {
            if (r[k] > 0.0f) {
                last_pos = e + k;
                if (cand == INT_MAX && excl + pre[k] > t) cand = e + k;
            }
        }
    }
    #pragma unroll
    for (int off = 32; off > 0; off >>= 1) {
        cand = min(cand, __shfl_xor(cand, off, 64));
        last_pos = max(last_pos, __shfl_xor(last_pos, off, 64));
    }
    if (lane == 0) {
        sh.red_i[wave] = cand;
        sh.red_f[wave] = __int_as_float(last_pos);
    }
    __syncthreads();
    int y = INT_MAX, lp = -1;
    #pragma unroll
    for (int w = 0; w < kWaves; ++w) {
        y = min(y, sh.red_i[w]);
        lp = max(lp, __float_as_int(sh.red_f[w]));
    }
    __syncthreads();
    return y != INT_MAX ? y : lp;
}

// Wave 0: find the chunk where the running mass over chunks 0..C-1 first
// exceeds thr. mass(cc) gives chunk cc's mass. Returns (chunk, mass before it)
// in every lane; chunk -1 if there is no mass.
template <typename F>
__device__ void chunk_crossing(int C, double thr, F mass, int& chunk, double& base) {
    const int lane = threadIdx.x & 63;
    const int per = (C + 63) / 64;
    const int a0 = min(lane * per, C), a1 = min(a0 + per, C);
    double acc = 0.0;
    for (int cc = a0; cc < a1; ++cc) acc += mass(cc);
    const double incl = wave_incl_scan(acc, lane);
    const double prev = __shfl_up(incl, 1, 64);
    const unsigned long long hit = __ballot(incl > thr);
    const int lane_star = hit ? (__ffsll((long long)hit) - 1) : 63;
    chunk = -1;
    base = 0.0;
    if (lane == lane_star) {
        double b = lane ? prev : 0.0;
        int found = -1, last = -1;
        double b_last = 0.0;
        for (int cc = a0; cc < a1; ++cc) {
            const double m = mass(cc);
            if (m > 0.0) {
                last = cc;
                b_last = b;
                if (b + m > thr) {
                    found = cc;
                    break;
                }
            }
            b += m;
        }
        if (found < 0) {
            found = last;
            b = b_last;
        }
        chunk = found;
        base = b;
    }
    chunk = __shfl(chunk, lane_star, 64);
    base = __shfl(base, lane_star, 64);
}

// ------------------------------------------------------ request outputs --

// Control lane: team (b, i) is complete (its result word is stored). The team
// completing last for request b writes the request's outputs and resets the
// request's counters for the next call.
template <bool kGreedy>
__device__ void team_complete(const Params& P, int b, int k) {
    drain();
    const unsigned old = add32(&P.req_count[b * kReqStride], 1u);
    if (old != (unsigned)k) return;
    const unsigned fr = ld32(&P.req_first[b * kReqStride]);
    const int j = fr < (unsigned)k ? (int)fr : k;
    const int y = (int)(unsigned)ld64(&P.result[(size_t)b * (P.K + 1) + j]);
    const int K = P.K;
    P.out_nacc[b] = j;
    for (int t = 0; t <= K; ++t) {
        int32_t v = -1;
        if (t < j) v = P.tokens[(size_t)b * K + t];
        else if (t == j) v = y;
        P.out_tokens[(size_t)b * (K + 1) + t] = v;
    }
    for (int t = kGreedy ? 0 : k; t < K; ++t) {
        if (P.out_p) P.out_p[(size_t)b * K + t] = NAN;
        if (P.out_q) P.out_q[(size_t)b * K + t] = NAN;
    }
    // Every unit of every team of this request has arrived: reset the teams'
    // counters (phase words carry the call epoch and need no reset).
    for (int t = 0; t <= k; ++t) {
        unsigned* tw = P.team + ((size_t)b * (K + 1) + t) * kTeamWords;
        st32(tw + TW_ARRIVE, 0u);
        st32(tw + TW_ARRIVE2, 0u);
    }
    st32(&P.req_count[b * kReqStride], 0u);
    st32(&P.req_first[b * kReqStride], kNoReject);
}

// ------------------------------------------------------------ leader work --

// Control wave, greedy: merge the chunk argmaxes of target row i, decide,
// complete the team.
__device__ void leader_greedy(const Params& P, int b, int i, int k, int tr) {
    const int lane = threadIdx.x & 63;
    const int C = P.C;
    float bv = -INFINITY;
    int bi = INT_MAX;
    for (int cc = lane; cc < C; cc += 64) {
        const unsigned long long w = ld64(&P.part[((size_t)tr * C + cc) * kPartWords]);
        const float v = __uint_as_float((unsigned)(w >> 32));
        const int idx = (int)(unsigned)w;
        if (better_arg(v, idx, bv, bi)) {
            bv = v;
            bi = idx;
        }
    }
    #pragma unroll
    for (int off = 32; off > 0; off >>= 1) {
        const float ov = __shfl_xor(bv, off, 64);
        const int oi = __shfl_xor(bi, off, 64);
        if (better_arg(ov, oi, bv, bi)) {
            bv = ov;
            bi = oi;
        }
    }
    if (lane == 0) {
        const int best = bi == INT_MAX ? 0 : bi;      // an all -inf row: index 0
        bool accept = true;
        if (i < k) {
            const int x = P.tokens[(size_t)b * P.K + i];
            const bool valid = x >= 0 && x < P.V;
            if (!valid) atomicOr(P.status, SV_FLAG_BAD_TOKEN);
            accept = valid && x == best;
            if (!accept) {
                __hip_atomic_fetch_min(&P.req_first[b * kReqStride], (unsigned)i,
                                       __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            }
        }
        st64(&P.result[tr], ((unsigned long long)(accept ? 1u : 0u) << 32) | (unsigned)best);
        team_complete<true>(P, b, k);
    }
}

// Control wave, sampled: merge the chunk statistics of target (and drafter)
// row i; for a drafted position take the accept decision and publish the
// normalisers; for the bonus position locate the chunk of the bonus draw and
// leave its element scan to the data waves (pend_bonus).
template <typename E>
__device__ void leader_sampled(const Params& P, Shared& sh, int b, int i, int k, int tr) {
    const int lane = threadIdx.x & 63;
    const int C = P.C;
    const int K = P.K;
    const E* target = static_cast<const E*>(P.target);
    const E* draft = static_cast<const E*>(P.draft);
    const unsigned long long* part = P.part + (size_t)tr * C * kPartWords;
    // Merge: M = max of chunk maxima, S = sum of S_c 2^((M_c - M) c).
    float mt = -INFINITY, md = -INFINITY;
    for (int cc = lane; cc < C; cc += 64) {
        const unsigned long long w = ld64(const_cast<unsigned long long*>(&part[cc * kPartWords]));
        mt = fmaxf(mt, __uint_as_float((unsigned)(w >> 32)));
        md = fmaxf(md, __uint_as_float((unsigned)w));
    }
    mt = wave_max(mt);
    md = wave_max(md);
    double st = 0.0, sd = 0.0;
    for (int cc = lane; cc < C; cc += 64) {
        unsigned long long* pw = const_cast<unsigned long long*>(&part[cc * kPartWords]);
        const unsigned long long w = ld64(pw);
        const double s1 = as_f64(ld64(pw + 1));
        const double s2 = as_f64(ld64(pw + 2));
        const float m1 = __uint_as_float((unsigned)(w >> 32));
        const float m2 = __uint_as_float((unsigned)w);
        if (s1 > 0.0) st += s1 * exp2(((double)m1 - (double)mt) * P.c64);
        if (s2 > 0.0) sd += s2 * exp2(((double)m2 - (double)md) * P.c64);
    }
    st = wave_sum(st);
    sd = wave_sum(sd);
    if (i < k) {
        if (lane == 0) {
            const int x = P.tokens[(size_t)b * K + i];
            const bool valid = x >= 0 && x < P.V;
            if (!valid) atomicOr(P.status, SV_FLAG_BAD_TOKEN);
            double px = 0.0, qx = 0.0;
            if (valid) {
                const float zt = Elem<E>::one(target + ((size_t)b * (K + 1) + i) * (size_t)P.V + x);
                const float zd = Elem<E>::one(draft + ((size_t)b * K + i) * (size_t)P.V + x);
                px = exp2(((double)zt - (double)mt) * P.c64) / st;
                qx = exp2(((double)zd - (double)md) * P.c64) / sd;
            }
            const uint4 rw = philox4x32_10((uint32_t)b, (uint32_t)i, 0u, 0u, P.key0, P.key1);
            const bool accept = word_to_uniform(rw.x) * qx < px;
            if (P.out_p) P.out_p[(size_t)b * K + i] = (float)px;
            if (P.out_q) P.out_q[(size_t)b * K + i] = (float)qx;
            bool residual = false;
            if (!accept) {
                const unsigned old = __hip_atomic_fetch_min(
                    &P.req_first[b * kReqStride], (unsigned)i, __ATOMIC_RELAXED,
                    __HIP_MEMORY_SCOPE_AGENT);
                residual = (unsigned)i < old;          // earliest rejection so far
            }
            unsigned* tw = P.team + (size_t)tr * kTeamWords;
            st64(reinterpret_cast<unsigned long long*>(tw + TW_ST), as_u64(st));
            st64(reinterpret_cast<unsigned long long*>(tw + TW_SD), as_u64(sd));
            st32(tw + TW_MT, __float_as_uint(mt));
            st32(tw + TW_MD, __float_as_uint(md));
            drain();
            st32(tw + TW_PHASE, (P.epoch << 2) | PH_READY | (residual ? PH_RESIDUAL : 0u));
            if (!residual) {
                st64(&P.result[tr], ((unsigned long long)(accept ? 1u : 0u) << 32) | 0xFFFFFFFFull);
                team_complete<false>(P, b, k);
            }
        }
        return;
    }
    // Bonus position: needed only if nothing was rejected so far.
    unsigned fr = 0;
    if (lane == 0) fr = ld32(&P.req_first[b * kReqStride]);
    fr = __shfl(fr, 0, 64);
    int go = 0;
    if (fr == kNoReject && st > 0.0) {
        const uint4 rw = philox4x32_10((uint32_t)b, (uint32_t)k, 0u, 0u, P.key0, P.key1);
        const double u = word_to_uniform(rw.y);
        const double inv = 1.0 / st;
        auto mass = [&](int cc) -> double {
            unsigned long long* pw = const_cast<unsigned long long*>(&part[cc * kPartWords]);
            const double s1 = as_f64(ld64(pw + 1));
            const float m1 = __uint_as_float((unsigned)(ld64(pw) >> 32));
            return s1 > 0.0 ? s1 * exp2(((double)m1 - (double)mt) * P.c64) * inv : 0.0;
        };
        double total = 0.0;
        for (int cc = lane; cc < C; cc += 64) total += mass(cc);
        total = wave_sum(total);
        int chunk;
        double base;
        chunk_crossing(C, u * total, mass, chunk, base);
        if (chunk >= 0) {
            go = 1;
            if (lane == 0) {
                sh.bonus_b = b;
                sh.bonus_k = k;
                sh.bonus_tr = tr;
                sh.bonus_chunk = chunk;
                sh.bonus_mt = mt;
                sh.bonus_ist = (float)inv;
                sh.bonus_thr = u * total - base;
            }
        }
    }
    if (lane == 0) {
        sh.pend_bonus = go;
        if (!go) {
            st64(&P.result[tr], (1ull << 32) | 0xFFFFFFFFull);
            team_complete<false>(P, b, k);
        }
    }
}

// Control wave: all chunks of a residual team published their residual mass;
// scan the residual CDF over chunks and leave the element scan of the chunk
// holding the threshold to the data waves (pend_resid).
template <typename E>
__device__ void residual_locate(const Params& P, Shared& sh, int b, int i, int k, int tr,
                                double st, float mt, float md, float ist, float isd) {
    const int lane = threadIdx.x & 63;
    const int C = P.C;
    const unsigned long long* part = P.part + (size_t)tr * C * kPartWords;
    const uint4 rw = philox4x32_10((uint32_t)b, (uint32_t)i, 0u, 0u, P.key0, P.key1);
    const double u_s = word_to_uniform(rw.y);
    auto rmass = [&](int cc) -> double {
        const double v = as_f64(ld64(const_cast<unsigned long long*>(&part[cc * kPartWords + 3])));
        return v > 0.0 ? v : 0.0;
    };
    double total = 0.0;
    for (int cc = lane; cc < C; cc += 64) total += rmass(cc);
    total = wave_sum(total);
    int chunk = -1;
    double base = 0.0;
    int residual = 1;
    if (total > 0.0) chunk_crossing(C, u_s * total, rmass, chunk, base);
    if (chunk < 0) {
        // The residual kept no mass (rounding only): draw from p_i.
        residual = 0;
        const double inv = 1.0 / st;
        auto pmass = [&](int cc) -> double {
            unsigned long long* pw = const_cast<unsigned long long*>(&part[cc * kPartWords]);
            const double s1 = as_f64(ld64(pw + 1));
            const float m1 = __uint_as_float((unsigned)(ld64(pw) >> 32));
            return s1 > 0.0 ? s1 * exp2(((double)m1 - (double)mt) * P.c64) * inv : 0.0;
        };
        total = 0.0;
        for (int cc = lane; cc < C; cc += 64) total += pmass(cc);
        total = wave_sum(total);
        chunk_crossing(C, u_s * total, pmass, chunk, base);
    }
    if (lane == 0) {
        sh.pend_resid = 1;
        sh.resid_b = b;
        sh.resid_i = i;
        sh.resid_k = k;
        sh.resid_tr = tr;
        sh.resid_mt = mt;
        sh.resid_md = md;
        sh.resid_ist = ist;
        sh.resid_isd = isd;
        sh.scan_chunk = chunk;
        sh.scan_residual = residual;
        sh.scan_thr = u_s * total - base;
    }
}

// ---------------------------------------------------------- main kernel --

// Coordinates of a work unit (uniform across the workgroup).
struct Unit {
    int u;         // unit index, -1: none
    int b, i, k, c;
    int tr;        // team record index b * (K + 1) + i
    int e0, n;     // chunk start and length (elements)
    bool has_d;    // drafted position in sampled mode: the drafter row is read too
};

__device__ __forceinline__ Unit decode_unit(const Params& P, const int* off, int u, int U,
                                            bool greedy) {
    Unit d;
    d.u = u < U ? u : -1;
    d.b = d.i = d.k = d.c = d.tr = d.e0 = d.n = 0;
    d.has_d = false;
    if (d.u < 0) return d;
    int lo_b = 0, hi_b = P.B;                      // largest b with off[b] <= u
    while (hi_b - lo_b > 1) {
        const int mid = (lo_b + hi_b) >> 1;
        if (off[mid] <= u) lo_b = mid; else hi_b = mid;
    }
    d.b = lo_b;
    const int local = u - off[d.b];
    d.k = (off[d.b + 1] - off[d.b]) / P.C - 1;
    d.i = local / P.C;
    d.c = local - d.i * P.C;
    d.tr = d.b * (P.K + 1) + d.i;
    d.e0 = d.c * P.CE;
    d.n = min(P.CE, P.V - d.e0);
    d.has_d = !greedy && d.i < d.k;
    return d;
}

// Data waves: issue the 16-byte loads of a unit into registers (no wait).
template <typename E, bool kVec>
__device__ __forceinline__ void issue_loads(const Params& P, const Unit& d, int dt,
                                            uint4 (&gt)[kG], uint4 (&gd)[kG]) {
    constexpr int W = Elem<E>::W;
    const E* target = static_cast<const E*>(P.target);
    const E* draft = static_cast<const E*>(P.draft);
    const E* bt = target + ((size_t)d.b * (P.K + 1) + d.i) * (size_t)P.V + d.e0;
    const E* bd = d.has_d ? draft + ((size_t)d.b * P.K + d.i) * (size_t)P.V + d.e0 : nullptr;
    const bool vt = aligned16(bt);
    const bool vd = d.has_d && aligned16(bd);
    #pragma unroll
    for (int j = 0; j < kG; ++j) {
        const int e = (dt + j * kDataThreads) * W;
        gt[j] = e < d.n ? load_group<E, kVec>(bt, e, d.n, vt) : neg_group<E>();
        gd[j] = (d.has_d && e < d.n) ? load_group<E, kVec>(bd, e, d.n, vd) : neg_group<E>();
    }
}

// Block-wide (max, lowest index) merge; every thread gets the result.
__device__ __forceinline__ void block_argmax(Shared& sh, float& bv, int& bi) {
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    #pragma unroll
    for (int o = 32; o > 0; o >>= 1) {
        const float ov = __shfl_xor(bv, o, 64);
        const int oi = __shfl_xor(bi, o, 64);
        if (better_arg(ov, oi, bv, bi)) {
            bv = ov;
            bi = oi;
        }
    }
    if (lane == 0) {
        sh.red_f[wave] = bv;
        sh.red_i[wave] = bi;
    }
    __syncthreads();
    #pragma unroll
    for (int w = 0; w < kWaves; ++w) {
        if (better_arg(sh.red_f[w], sh.red_i[w], bv, bi)) {
            bv = sh.red_f[w];
            bi = sh.red_i[w];
        }
    }
}

// Deferred draws left by the previous round (whole workgroup): the element
// scan of the one chunk that holds the bonus or the residual threshold. The
// control wave's lane 0 stores the result and completes the team.
template <typename E, bool kVec, bool kCtrl>
__device__ __forceinline__ void pending_draws(const Params& P, Shared& sh) {
    const int K = P.K;
    if (sh.pend_bonus) {
        const E* target = static_cast<const E*>(P.target);
        const int chunk = sh.bonus_chunk;
        const int e0 = chunk * P.CE;
        const int n = min(P.CE, P.V - e0);
        const E* rt = target + ((size_t)sh.bonus_b * (K + 1) + sh.bonus_k) * (size_t)P.V + e0;
        const int o = chunk_scan<E, kVec>(sh, rt, nullptr, n, sh.bonus_mt, sh.bonus_ist, 0.0f,
                                          0.0f, P.c32, sh.bonus_thr);
        if (kCtrl && threadIdx.x == 0) {
            const int y = o < 0 ? 0 : e0 + o;
            st64(&P.result[sh.bonus_tr], (1ull << 32) | (unsigned)y);
            team_complete<false>(P, sh.bonus_b, sh.bonus_k);
            sh.pend_bonus = 0;
        }
        __syncthreads();
    }
    if (sh.pend_resid) {
        const E* target = static_cast<const E*>(P.target);
        const E* draft = static_cast<const E*>(P.draft);
        const int chunk = sh.scan_chunk;
        int y = 0;
        if (chunk >= 0) {
            const int e0 = chunk * P.CE;
            const int n = min(P.CE, P.V - e0);
            const E* rt = target + ((size_t)sh.resid_b * (K + 1) + sh.resid_i) * (size_t)P.V + e0;
            const E* rd = sh.scan_residual
                              ? draft + ((size_t)sh.resid_b * K + sh.resid_i) * (size_t)P.V + e0
                              : nullptr;
            const int o = chunk_scan<E, kVec>(sh, rt, rd, n, sh.resid_mt, sh.resid_ist,
                                              sh.resid_md, sh.resid_isd, P.c32, sh.scan_thr);
            y = o < 0 ? 0 : e0 + o;
        }
        if (kCtrl && threadIdx.x == 0) {
            st64(&P.result[sh.resid_tr], (unsigned)y);
            team_complete<false>(P, sh.resid_b, sh.resid_k);
            sh.pend_resid = 0;
        }
        __syncthreads();
    }
}

// Control wave: the loop of a workgroup's control wave. It mirrors the data
// waves' loop barrier for barrier (every branch below depends only on values
// the whole workgroup shares), contributes neutral values to the block
// reductions, and does all synchronisation with other workgroups.
template <typename E, bool kGreedy, bool kVec>
__device__ __forceinline__ void control_loop(const Params& P, Shared& sh, const int* off) {
    const int lane = threadIdx.x & 63;
    const int C = P.C;
    const int U = off[P.B];
    const int G = gridDim.x;
    const unsigned ep = P.epoch & 0x3FFFFFFFu;
    Unit cur = decode_unit(P, off, blockIdx.x, U, kGreedy);
    Unit prev;
    prev.u = -1;
    for (;;) {
        // Read the parked unit's team phase early; the draws below hide the latency.
        unsigned ph = 0;
        if (lane == 0 && prev.u >= 0) ph = ld32(P.team + (size_t)prev.tr * kTeamWords + TW_PHASE);

        pending_draws<E, kVec, true>(P, sh);

        if (prev.u >= 0) {
            // Wait for the parked unit's team decision.
            if (lane == 0) {
                unsigned* tw = P.team + (size_t)prev.tr * kTeamWords;
                for (unsigned it = 0; (ph >> 2) != ep && it < kSpinLimit; ++it) {
                    __builtin_amdgcn_s_sleep(2);
                    ph = ld32(tw + TW_PHASE);
                }
                if ((ph >> 2) != ep) {
                    atomicOr(P.status, SV_FLAG_SYNC_TIMEOUT);
                    ph = PH_READY;
                }
                sh.phase = ph;
                if (ph & PH_RESIDUAL) {
                    sh.nst = as_f64(ld64(reinterpret_cast<unsigned long long*>(tw + TW_ST)));
                    sh.nsd = as_f64(ld64(reinterpret_cast<unsigned long long*>(tw + TW_SD)));
                    sh.nmt = __uint_as_float(ld32(tw + TW_MT));
                    sh.nmd = __uint_as_float(ld32(tw + TW_MD));
                }
            }
            __syncthreads();
            if (sh.phase & PH_RESIDUAL) {
                // The request's earliest rejection: publish the parked chunk's
                // residual mass; the last chunk to do so locates the draw.
                const double2 R = block_sum2(sh, 0.0, 0.0);
                int last = 0;
                if (lane == 0) {
                    st64(P.part + ((size_t)prev.tr * C + prev.c) * kPartWords + 3, as_u64(R.x));
                    drain();
                    const unsigned old = add32(&P.team[(size_t)prev.tr * kTeamWords + TW_ARRIVE2], 1u);
                    last = old == (unsigned)C - 1;
                }
                last = __shfl(last, 0, 64);
                if (last) {
                    const float ist = (float)(1.0 / sh.nst), isd = (float)(1.0 / sh.nsd);
                    residual_locate<E>(P, sh, prev.b, prev.i, prev.k, prev.tr, sh.nst, sh.nmt,
                                       sh.nmd, ist, isd);
                }
            }
            prev.u = -1;
        }

        if (cur.u < 0) {
            __syncthreads();
            if (sh.pend_bonus || sh.pend_resid) continue;
            break;
        }

        // The current unit's chunk statistics (the data waves hold the data).
        unsigned long long w0;
        double s_t = 0.0, s_d = 0.0;
        if (kGreedy) {
            float bv = -INFINITY;
            int bi = INT_MAX;
            block_argmax(sh, bv, bi);
            w0 = ((unsigned long long)__float_as_uint(bv) << 32) | (unsigned)bi;
        } else {
            const float2 M = block_max2(sh, -INFINITY, -INFINITY);
            const double2 S = block_sum2(sh, 0.0, 0.0);
            s_t = S.x;
            s_d = S.y;
            w0 = ((unsigned long long)__float_as_uint(M.x) << 32) | __float_as_uint(M.y);
        }

        // Publish, arrive; the last arrival of a team leads it.
        int lead = 0;
        if (lane == 0) {
            unsigned long long* pw = P.part + ((size_t)cur.tr * C + cur.c) * kPartWords;
            st64(pw, w0);
            if (!kGreedy) {
                st64(pw + 1, as_u64(s_t));
                st64(pw + 2, as_u64(s_d));
            }
            drain();
            const unsigned old = add32(&P.team[(size_t)cur.tr * kTeamWords + TW_ARRIVE], 1u);
            lead = old == (unsigned)C - 1;
        }
        lead = __shfl(lead, 0, 64);
        if (lead) {
            if (kGreedy) {
                leader_greedy(P, cur.b, cur.i, cur.k, cur.tr);
            } else {
                leader_sampled<E>(P, sh, cur.b, cur.i, cur.k, cur.tr);
            }
        }
        __syncthreads();
        if (cur.has_d) prev = cur;
        cur = decode_unit(P, off, cur.u + G, U, kGreedy);
    }
}

// Data waves: stream units through registers, reduce them, park them in LDS.
template <typename E, bool kGreedy, bool kVec>
__device__ __forceinline__ void data_loop(const Params& P, Shared& sh, const int* off,
                                          uint4* stash) {
    constexpr int W = Elem<E>::W;
    const int dt = threadIdx.x - 64;               // data thread index
    const int U = off[P.B];
    const int G = gridDim.x;
    const float cs = P.c32;

    uint4 gt[kG], gd[kG];
    Unit cur = decode_unit(P, off, blockIdx.x, U, kGreedy);
    if (cur.u >= 0) issue_loads<E, kVec>(P, cur, dt, gt, gd);
    bool have_prev = false;

    for (;;) {
        pending_draws<E, kVec, false>(P, sh);

        if (have_prev) {
            __syncthreads();                       // the control wave has the parked team's phase
            if (sh.phase & PH_RESIDUAL) {
                const float mt = sh.nmt, md = sh.nmd;
                const float ist = (float)(1.0 / sh.nst), isd = (float)(1.0 / sh.nsd);
                float lr = 0.0f;
                #pragma unroll 1
                for (int j = 0; j < kG; ++j) {
                    // Each lane reads back only the groups it parked itself.
                    const uint4 a = stash[(0 * kG + j) * kDataThreads + dt];
                    const uint4 d = stash[(1 * kG + j) * kDataThreads + dt];
                    float r[W];
                    #pragma unroll
                    for (int kk = 0; kk < W; ++kk) {
                        const float pv = fast_exp2((Elem<E>::at(a, kk) - mt) * cs) * ist;
                        const float qv = fast_exp2((Elem<E>::at(d, kk) - md) * cs) * isd;
                        r[kk] = fmaxf(0.0f, pv - qv);
                    }
                    #pragma unroll
                    for (int h = W / 2; h > 0; h >>= 1) {
                        #pragma unroll
                        for (int kk = 0; kk < h; ++kk) r[kk] += r[kk + h];
                    }
                    lr += r[0];
                }
                (void)block_sum2(sh, (double)lr, 0.0);
            }
            have_prev = false;
        }

        if (cur.u < 0) {
            __syncthreads();
            if (sh.pend_bonus || sh.pend_resid) continue;
            break;
        }

        // Reduce the current unit to its chunk statistics.
        if (kGreedy) {
            float bv = -INFINITY;
            int bi = INT_MAX;
            #pragma unroll
            for (int j = 0; j < kG; ++j) {
                #pragma unroll
                for (int kk = 0; kk < W; ++kk) {
                    const float v = Elem<E>::at(gt[j], kk);
                    if (v > bv) {                  // a lane's elements go up in index order
                        bv = v;
                        bi = cur.e0 + (dt + j * kDataThreads) * W + kk;
                    }
                }
            }
            block_argmax(sh, bv, bi);
        } else {
            float mt = -INFINITY, md = -INFINITY;
            #pragma unroll
            for (int j = 0; j < kG; ++j) {
                #pragma unroll
                for (int kk = 0; kk < W; ++kk) {
                    mt = fmaxf(mt, Elem<E>::at(gt[j], kk));
                    md = fmaxf(md, Elem<E>::at(gd[j], kk));
                }
            }
            // Opaque raw registers: the exp pass converts them again rather
            // than keeping every converted float alive across the barrier.
            #pragma unroll
            for (int j = 0; j < kG; ++j) {
                asm volatile("" : "+v"(gt[j].x), "+v"(gt[j].y), "+v"(gt[j].z), "+v"(gt[j].w));
                asm volatile("" : "+v"(gd[j].x), "+v"(gd[j].y), "+v"(gd[j].z), "+v"(gd[j].w));
            }
            const float2 M = block_max2(sh, mt, md);
            float lt = 0.0f, ld = 0.0f;
            if (M.x != -INFINITY) {
                #pragma unroll
                for (int j = 0; j < kG; ++j) {
                    float e[W];
                    #pragma unroll
                    for (int kk = 0; kk < W; ++kk) e[kk] = fast_exp2((Elem<E>::at(gt[j], kk) - M.x) * cs);
                    #pragma unroll
                    for (int h = W / 2; h > 0; h >>= 1) {
                        #pragma unroll
                        for (int kk = 0; kk < h; ++kk) e[kk] += e[kk + h];
                    }
                    lt += e[0];
                }
            }
            if (cur.has_d && M.y != -INFINITY) {
                #pragma unroll
                for (int j = 0; j < kG; ++j) {
                    float e[W];
                    #pragma unroll
                    for (int kk = 0; kk < W; ++kk) e[kk] = fast_exp2((Elem<E>::at(gd[j], kk) - M.y) * cs);
                    #pragma unroll
                    for (int h = W / 2; h > 0; h >>= 1) {
                        #pragma unroll
                        for (int kk = 0; kk < h; ++kk) e[kk] += e[kk + h];
                    }
                    ld += e[0];
                }
            }
            (void)block_sum2(sh, (double)lt, (double)ld);
        }

        // Park the unit, start streaming the next one.
        const Unit nxt = decode_unit(P, off, cur.u + G, U, kGreedy);
        if (cur.has_d) {
            #pragma unroll
            for (int j = 0; j < kG; ++j) {
                stash[(0 * kG + j) * kDataThreads + dt] = gt[j];
                stash[(1 * kG + j) * kDataThreads + dt] = gd[j];
            }
        }
        if (nxt.u >= 0) issue_loads<E, kVec>(P, nxt, dt, gt, gd);
        __syncthreads();                           // the control wave has published and led
        if (cur.has_d) have_prev = true;
        cur = nxt;
    }
}

template <typename E, bool kGreedy, bool kVec>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(4))) void verify_kernel(Params P) {
    extern __shared__ __align__(16) unsigned char dyn_smem[];
    __shared__ Shared sh;
    // Dynamic LDS: the parked unit (sampled mode), then request unit offsets.
    uint4* stash = reinterpret_cast<uint4*>(dyn_smem);
    int* off = reinterpret_cast<int*>(dyn_smem + (kGreedy ? 0 : (size_t)2 * kG * kDataThreads * 16));

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int B = P.B, K = P.K, C = P.C;

    // Prologue: every workgroup scans the budgets into per-request unit offsets.
    {
        const int per = (B + kThreads - 1) / kThreads;
        const int b0 = min(tid * per, B), b1 = min(b0 + per, B);
        int local = 0;
        bool bad = false;
        for (int b = b0; b < b1; ++b) {
            int k = P.budgets[b];
            if (k < 0 || k > K) {
                bad = true;
                k = k < 0 ? 0 : K;
            }
            local += (k + 1) * C;
        }
        if (bad && blockIdx.x == 0) atomicOr(P.status, SV_FLAG_BAD_BUDGET);
        int incl = local;
        #pragma unroll
        for (int o = 1; o < 64; o <<= 1) {
            const int v = __shfl_up(incl, o, 64);
            if (lane >= o) incl += v;
        }
        if (lane == 63) sh.red_i[wave] = incl;
        __syncthreads();
        int run = incl - local;
        for (int w = 0; w < wave; ++w) run += sh.red_i[w];
        for (int b = b0; b < b1; ++b) {
            off[b] = run;
            int k = P.budgets[b];
            k = k < 0 ? 0 : (k > K ? K : k);
            run += (k + 1) * C;
        }
        if (tid == kThreads - 1) off[B] = run;
        if (tid == 0) {
            sh.pend_bonus = 0;
            sh.pend_resid = 0;
        }
        __syncthreads();
    }

    // Wave specialisation: the branch is uniform per wave, and the two loops
    // execute the same sequence of barriers.
    if (__builtin_amdgcn_readfirstlane(wave) == 0) {
        control_loop<E, kGreedy, kVec>(P, sh, off);
    } else {
        data_loop<E, kGreedy, kVec>(P, sh, off, stash);
    }
}

// Philox blocks as the verifier draws them, for checking the generator.
__global__ void philox_words_kernel(uint32_t k0, uint32_t k1, int B, int P, uint32_t* out) {
    const long long n = (long long)B * P;
    for (long long t = blockIdx.x * (long long)blockDim.x + threadIdx.x; t < n;
         t += (long long)gridDim.x * blockDim.x) {
        const uint32_t b = (uint32_t)(t / P), i = (uint32_t)(t % P);
        const uint4 r = philox4x32_10(b, i, 0u, 0u, k0, k1);
        out[t * 4 + 0] = r.x;
        out[t * 4 + 1] = r.y;
        out[t * 4 + 2] = r.z;
        out[t * 4 + 3] = r.w;
    }
}

// ------------------------------------------------------------- host side --

constexpr uint32_t kMagic = 0x53505643u;   // live context marker

int elems_per_group(int dtype) { return dtype == SV_DTYPE_BF16 ? 8 : 4; }

int chunk_elems(int dtype) { return kDataThreads * kG * elems_per_group(dtype); }

int chunks_for(int vocab, int dtype) {
    const int ce = chunk_elems(dtype);
    return (vocab + ce - 1) / ce;
}

size_t dyn_smem_bytes(int B, bool greedy) {
    return (greedy ? 0 : (size_t)2 * kG * kDataThreads * 16) + (size_t)(B + 1) * sizeof(int);
}

}  // namespace

struct spec_verify_ctx {
    uint32_t magic;
    int device, max_batch, max_k, vocab, dtype;
    int C, CE;
    int cus;
    void* ws;
    unsigned long long* part;
    unsigned* team;
    unsigned long long* result;
    unsigned* req_count;
    unsigned* req_first;
    unsigned* status;
    unsigned calls;                // calls made so far (phase-word epochs)
    // occupancy cache: dynamic LDS bytes -> resident workgroups per CU, per kernel
    size_t occ_smem[8];
    int occ_val[8];
};

namespace {

template <typename E, bool G, bool Vv>
int occupancy_of(spec_verify_ctx* ctx, int slot, size_t smem) {
    if (ctx->occ_smem[slot] == smem && ctx->occ_val[slot] > 0) return ctx->occ_val[slot];
    int n = 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, verify_kernel<E, G, Vv>, kThreads, smem) !=
            hipSuccess ||
        n < 1) {
        n = 1;
    }
    ctx->occ_smem[slot] = smem;
    ctx->occ_val[slot] = n;
    return n;
}

// Launch shape: every workgroup resident (grid = CUs x occupancy); the
// schedule needs at least as many workgroups as a team has members.
template <typename E, bool G, bool Vv>
int launch(spec_verify_ctx* ctx, Params& p, hipStream_t stream) {
    const int slot = (std::is_same<E, uint16_t>::value ? 4 : 0) + (G ? 2 : 0) + (Vv ? 1 : 0);
    const size_t smem = dyn_smem_bytes(p.B, G);
    const int occ = occupancy_of<E, G, Vv>(ctx, slot, smem);
    const long long grid = (long long)ctx->cus * occ;
    if (grid < (long long)p.C) return SV_ERR_ARG;   // a team would not fit
    hipLaunchKernelGGL((verify_kernel<E, G, Vv>), dim3((unsigned)grid), dim3(kThreads), smem, stream,
                       p);
    return hipGetLastError() == hipSuccess ? SV_OK : SV_ERR_HIP;
}

bool aligned_to(const void* p, size_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

}  // namespace

extern "C" {

const char* spec_verify_strerror(int code) {
    switch (code) {
        case SV_OK: return "ok";
        case SV_ERR_NULL: return "a required pointer is NULL";
        case SV_ERR_ARG: return "a scalar argument is out of range";
        case SV_ERR_DTYPE: return "unknown logit storage type";
        case SV_ERR_ALIGN: return "a pointer is not aligned to its element size";
        case SV_ERR_HIP: return "HIP runtime error";
        case SV_ERR_NOMEM: return "device workspace allocation failed";
        case SV_ERR_STATE: return "NULL or freed context";
        default: return "unknown status code";
    }
}

int spec_verify_chunks(int vocab, int dtype) {
    if (dtype != SV_DTYPE_F32 && dtype != SV_DTYPE_BF16) return SV_ERR_DTYPE;
    if (vocab < 1 || vocab > SV_MAX_VOCAB) return SV_ERR_ARG;
    return chunks_for(vocab, dtype);
}

int spec_verify_check_args(int max_batch, int max_k, int vocab, int dtype,
                           const void* target_logits, const void* draft_logits,
                           const void* draft_tokens, const void* budgets, int B, int K,
                           float temperature, const void* out_tokens,
                           const void* out_num_accepted, const void* out_p_draft,
                           const void* out_q_draft) {
    if (dtype != SV_DTYPE_F32 && dtype != SV_DTYPE_BF16) return SV_ERR_DTYPE;
    if (max_batch < 1 || max_batch > SV_MAX_BATCH || max_k < 0 || max_k > SV_MAX_K ||
        vocab < 1 || vocab > SV_MAX_VOCAB) {
        return SV_ERR_ARG;
    }
    if (B < 0 || B > max_batch || K < 0 || K > max_k) return SV_ERR_ARG;
    if (!std::isfinite(temperature) || temperature < 0.0f) return SV_ERR_ARG;
    if (B == 0) return SV_OK;
    const bool greedy = temperature == 0.0f;
    if (!target_logits || !budgets || !out_tokens || !out_num_accepted) return SV_ERR_NULL;
    if (K > 0 && !draft_tokens) return SV_ERR_NULL;
    if (!greedy && K > 0 && !draft_logits) return SV_ERR_NULL;
    const size_t es = dtype == SV_DTYPE_BF16 ? 2 : 4;
    if (!aligned_to(target_logits, es) || (draft_logits && !aligned_to(draft_logits, es)) ||
        (draft_tokens && !aligned_to(draft_tokens, 4)) || !aligned_to(budgets, 4) ||
        !aligned_to(out_tokens, 4) || !aligned_to(out_num_accepted, 4) ||
        (out_p_draft && !aligned_to(out_p_draft, 4)) ||
        (out_q_draft && !aligned_to(out_q_draft, 4))) {
        return SV_ERR_ALIGN;
    }
    return SV_OK;
}

int spec_verify_init(spec_verify_ctx** out, int device, int max_batch, int max_k, int vocab,
                     int dtype) {
    if (!out) return SV_ERR_NULL;
    *out = nullptr;
    if (dtype != SV_DTYPE_F32 && dtype != SV_DTYPE_BF16) return SV_ERR_DTYPE;
    if (device < 0 || max_batch < 1 || max_batch > SV_MAX_BATCH || max_k < 0 ||
        max_k > SV_MAX_K || vocab < 1 || vocab > SV_MAX_VOCAB) {
        return SV_ERR_ARG;
    }
    int ndev = 0;
    if (hipGetDeviceCount(&ndev) != hipSuccess || device >= ndev) return SV_ERR_HIP;
    int prev = -1;
    if (hipGetDevice(&prev) != hipSuccess) return SV_ERR_HIP;
    if (hipSetDevice(device) != hipSuccess) return SV_ERR_HIP;

    spec_verify_ctx* c = new spec_verify_ctx();
    c->magic = kMagic;
    c->device = device;
    c->max_batch = max_batch;
    c->max_k = max_k;
    c->vocab = vocab;
    c->dtype = dtype;
    c->C = chunks_for(vocab, dtype);
    c->CE = chunk_elems(dtype);
    int rc = SV_OK;
    if (hipDeviceGetAttribute(&c->cus, hipDeviceAttributeMultiprocessorCount, device) !=
        hipSuccess) {
        rc = SV_ERR_HIP;
    }
    auto round256 = [](size_t x) { return (x + 255) / 256 * 256; };
    const size_t teams = (size_t)max_batch * (max_k + 1);
    const size_t part_bytes = round256(teams * c->C * kPartWords * 8);
    const size_t team_bytes = round256(teams * kTeamWords * 4);
    const size_t result_bytes = round256(teams * 8);
    const size_t req_bytes = round256((size_t)max_batch * kReqStride * 4);
    const size_t total = part_bytes + team_bytes + result_bytes + 2 * req_bytes + 256;
    if (rc == SV_OK && hipMalloc(&c->ws, total) != hipSuccess) {
        c->ws = nullptr;
        rc = SV_ERR_NOMEM;
    }
    if (rc == SV_OK) {
        unsigned char* w = static_cast<unsigned char*>(c->ws);
        size_t o = 0;
        c->part = reinterpret_cast<unsigned long long*>(w + o);
        o += part_bytes;
        c->team = reinterpret_cast<unsigned*>(w + o);
        o += team_bytes;
        c->result = reinterpret_cast<unsigned long long*>(w + o);
        o += result_bytes;
        c->req_count = reinterpret_cast<unsigned*>(w + o);
        o += req_bytes;
        c->req_first = reinterpret_cast<unsigned*>(w + o);
        o += req_bytes;
        c->status = reinterpret_cast<unsigned*>(w + o);
        if (hipMemset(c->ws, 0, total) != hipSuccess ||
            hipMemset(c->req_first, 0x7F, req_bytes) != hipSuccess ||
            hipDeviceSynchronize() != hipSuccess) {
            rc = SV_ERR_HIP;
        }
    }
    (void)hipSetDevice(prev);
    if (rc != SV_OK) {
        if (c->ws) (void)hipFree(c->ws);
        c->magic = 0;
        delete c;
        return rc;
    }
    *out = c;
    return SV_OK;
}

int spec_verify_run(spec_verify_ctx* ctx, const void* target_logits, const void* draft_logits,
                    const int32_t* draft_tokens, const int32_t* budgets, int B, int K,
                    float temperature, uint64_t seed, int32_t* out_tokens,
                    int32_t* out_num_accepted, float* out_p_draft, float* out_q_draft,
                    void* stream) {
    if (!ctx || ctx->magic != kMagic) return SV_ERR_STATE;
    const int rc = spec_verify_check_args(ctx->max_batch, ctx->max_k, ctx->vocab, ctx->dtype,
                                          target_logits, draft_logits, draft_tokens, budgets, B,
                                          K, temperature, out_tokens, out_num_accepted,
                                          out_p_draft, out_q_draft);
    if (rc != SV_OK) return rc;
    if (B == 0) return SV_OK;
    const bool greedy = temperature == 0.0f;

    Params p;
    std::memset(&p, 0, sizeof(p));
    p.target = target_logits;
    p.draft = greedy ? nullptr : draft_logits;
    p.tokens = draft_tokens;
    p.budgets = budgets;
    p.out_tokens = out_tokens;
    p.out_nacc = out_num_accepted;
    p.out_p = out_p_draft;
    p.out_q = out_q_draft;
    p.part = ctx->part;
    p.team = ctx->team;
    p.result = ctx->result;
    p.req_count = ctx->req_count;
    p.req_first = ctx->req_first;
    p.status = ctx->status;
    p.B = B;
    p.K = K;
    p.V = ctx->vocab;
    p.C = ctx->C;
    p.CE = ctx->CE;
    p.c64 = greedy ? 0.0 : kLog2e / (double)temperature;
    p.c32 = (float)p.c64;
    p.key0 = (uint32_t)(seed & 0xFFFFFFFFu);
    p.key1 = (uint32_t)(seed >> 32);
    ctx->calls = ctx->calls % 0x3FFFFFFFu + 1u;     // 1 .. 2^30 - 1, never 0
    p.epoch = ctx->calls;

    int prev = -1;
    if (hipGetDevice(&prev) != hipSuccess) return SV_ERR_HIP;
    if (prev != ctx->device && hipSetDevice(ctx->device) != hipSuccess) return SV_ERR_HIP;
    hipStream_t s = static_cast<hipStream_t>(stream);
    int r;
    // Vector-only loads when every row starts on a 16-byte boundary.
    const size_t es = ctx->dtype == SV_DTYPE_BF16 ? 2 : 4;
    const bool vec = aligned_to(target_logits, 16) &&
                     (greedy || K == 0 || aligned_to(draft_logits, 16)) &&
                     ((size_t)ctx->vocab * es) % 16 == 0;
    if (ctx->dtype == SV_DTYPE_BF16) {
        if (vec) {
            r = greedy ? launch<uint16_t, true, true>(ctx, p, s) : launch<uint16_t, false, true>(ctx, p, s);
        } else {
            r = greedy ? launch<uint16_t, true, false>(ctx, p, s) : launch<uint16_t, false, false>(ctx, p, s);
        }
    } else {
        if (vec) {
            r = greedy ? launch<float, true, true>(ctx, p, s) : launch<float, false, true>(ctx, p, s);
        } else {
            r = greedy ? launch<float, true, false>(ctx, p, s) : launch<float, false, false>(ctx, p, s);
        }
    }
    if (prev != ctx->device) (void)hipSetDevice(prev);
    return r;
}

int spec_verify_status(spec_verify_ctx* ctx, uint32_t* flags) {
    if (!ctx || ctx->magic != kMagic) return SV_ERR_STATE;
    if (!flags) return SV_ERR_NULL;
    int prev = -1;
    if (hipGetDevice(&prev) != hipSuccess) return SV_ERR_HIP;
    if (prev != ctx->device && hipSetDevice(ctx->device) != hipSuccess) return SV_ERR_HIP;
    int rc = SV_OK;
    unsigned v = 0;
    if (hipDeviceSynchronize() != hipSuccess ||
        hipMemcpy(&v, ctx->status, sizeof(v), hipMemcpyDeviceToHost) != hipSuccess ||
        hipMemset(ctx->status, 0, sizeof(unsigned)) != hipSuccess ||
        hipDeviceSynchronize() != hipSuccess) {
        rc = SV_ERR_HIP;
    }
    if (prev != ctx->device) (void)hipSetDevice(prev);
    *flags = v;
    return rc;
}

int spec_verify_philox_words(uint64_t seed, int B, int P, uint32_t* out_words, void* stream) {
    if (B < 0 || P < 0) return SV_ERR_ARG;
    if ((long long)B * P == 0) return SV_OK;
    if (!out_words) return SV_ERR_NULL;
    const long long n = (long long)B * P;
    const int threads = 256;
    long long blocks = (n + threads - 1) / threads;
    if (blocks > 65536) blocks = 65536;
    hipLaunchKernelGGL(philox_words_kernel, dim3((unsigned)blocks), dim3(threads), 0,
                       static_cast<hipStream_t>(stream), (uint32_t)(seed & 0xFFFFFFFFu),
                       (uint32_t)(seed >> 32), B, P, out_words);
    return hipGetLastError() == hipSuccess ? SV_OK : SV_ERR_HIP;
}

void spec_verify_free(spec_verify_ctx* ctx) {
    if (!ctx || ctx->magic != kMagic) return;
    int prev = -1;
    (void)hipGetDevice(&prev);
    if (prev != ctx->device) (void)hipSetDevice(ctx->device);
    (void)hipDeviceSynchronize();
    if (ctx->ws) (void)hipFree(ctx->ws);
    if (prev != ctx->device && prev >= 0) (void)hipSetDevice(prev);
    ctx->magic = 0;
    ctx->ws = nullptr;
    delete ctx;
}

}  // extern "C"
