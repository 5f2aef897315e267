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
//    into registers, all in flight at once, reduced per wave to the max and
//    sum of 2^((z - max) log2(e)/T) (sampled) or (max, lowest index)
//    (greedy), posted to LDS. Wave 0 is the control wave: it merges the
//    waves' statistics and publishes the chunk's partial record. The two
//    kinds of waves exchange tagged LDS messages, with no workgroup barrier
//    in the streaming loop.
//  * Sampled mode: every record word carries the call's epoch, so a record
//    is complete when all its words carry it. Every member of a team reads
//    the C records of its team once they are complete and takes the team's
//    accept decision itself (the same deterministic merge in every member);
//    no election and no counter sits between a chunk's statistics and its
//    team's decision. Meanwhile the drafted unit's data waits in a per-lane
//    LDS slot; on a rejection each member turns its parked chunk into its
//    residual mass max(0, p - q) and publishes it.
//  * The member holding chunk 0 keeps the books: p(x), q(x), the decision
//    word, and, for a rejection or a bonus position, a draw queued to the end
//    of its loop. There, once the earlier positions of the request are
//    decided, the draw is made only for the request's first rejection (or
//    the bonus position when none): residual CDF over chunks from the
//    published masses, then the whole workgroup re-reads the one chunk that
//    holds the threshold for the element-level scan.
//  * Greedy mode: the last arriver of a team (device-scope counter) merges
//    the chunk argmaxes and decides; no data is parked.
//  * Per request, the team that completes last writes the outputs.
//  * Waiting: inside the loop a workgroup waits only for the records of a
//    team it has already published to, and never while it holds an
//    unpublished unit; by induction on the unit index every record gets
//    written. Waits at the end of the loop depend only on work done inside
//    loops. Every wait is bounded (status flag on expiry) so the kernel
//    always drains.
//  * Synchronisation uses device-scope relaxed atomics (plus s_waitcnt where
//    a counter orders earlier stores), never release/acquire fences: those
//    write back and invalidate the whole L2.

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
constexpr int kMaxSub = 4;                     // sub-tiles per chunk
constexpr int kTeamWords = 32;                 // words per team record (128 bytes)
constexpr int kReqStride = 16;                 // words between request counters (64 bytes)
constexpr unsigned kSpinLimit = 1u << 20;      // bounded device-scope wait (~1 s)
constexpr unsigned kLdsSpinLimit = 1u << 26;   // bounded LDS mailbox wait (~3 s)

// Team record words.
constexpr int TW_ARRIVE = 0;    // greedy: units of the team that published their argmax
constexpr int TW_DEC = 2;       // 64-bit decision: (epoch << 32) | accepted (words 2-3)

// Unit record: 8 64-bit words.
//   sampled: word f = (value bits << 32) | epoch for the fp32 values
//            R_MT max of z_t, R_MD max of z_d, R_ST sum of 2^((z_t - M_t) c),
//            R_SD likewise, R_RES residual mass once the team has rejected
//   greedy:  word 0 = (max bits << 32) | lowest index of the max
constexpr int kRecWords = 8;
constexpr int R_MT = 0, R_MD = 1, R_ST = 2, R_SD = 3, R_RES = 4;
constexpr int kStatWords = 4;   // words R_MT..R_SD make a record complete
constexpr int kMaxChunks = 192; // chunks per row the team merge supports

// Decision posted to the data waves for a parked unit.
constexpr unsigned PH_ACCEPT = 1u;
constexpr unsigned PH_REJECT = 2u;              // data waves: publish the residual mass

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
    unsigned long long* rec;       // [B*(K+1)*C][kRecWords]
    unsigned* team;                // [B*(K+1)][kTeamWords]
    unsigned* result;              // [B*(K+1)]: drawn token of the team
    unsigned* req_count;           // [B][kReqStride]: teams completed
    int* tasks;                    // [G][task_cap]: deferred draws, 2 * team + is_bonus
    unsigned* status;              // 1 word
    int B, K, V;
    int C;                         // chunks per row
    int CE;                        // elements per chunk
    int task_cap;                  // task list entries per workgroup
    float c32;                     // log2(e) / T
    double c64;
    uint32_t key0, key1;
    unsigned epoch;                // call number (never 0): tags record and decision words
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

// Epoch-tagged 32-bit value.
__device__ __forceinline__ unsigned long long tagged(float v, unsigned ep) {
    return ((unsigned long long)__float_as_uint(v) << 32) | ep;
}
__device__ __forceinline__ float tag_val(unsigned long long w) {
    return __uint_as_float((unsigned)(w >> 32));
}
__device__ __forceinline__ bool tag_ok(unsigned long long w, unsigned ep) {
    return (unsigned)w == ep;
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

// Workgroup-local state. The streaming loop has no workgroup barrier: the
// data waves and the control wave exchange tagged messages through these
// mailboxes (a tag is written after its payload; LDS operations of one wave
// complete in order, so a reader that sees the tag sees the payload).
struct Shared {
    // Data wave -> control wave: a unit's per-wave statistics, by round parity.
    //   sampled: (max, sum of 2^((z - max) c)) of the target and drafter parts
    //   greedy:  (max, lowest index of the max) of the target part
    float st_mt[2][kDataWaves];
    float st_md[2][kDataWaves];
    double st_st[2][kDataWaves];
    double st_sd[2][kDataWaves];
    int st_idx[2][kDataWaves];
    int st_tag[2][kDataWaves];                   // round + 1
    int st_done[2];                              // control wave: round + 1 of the slot it read last
    // Control wave -> data waves: the parked unit's decision and the team's
    // normalisers, posted in round r (tag r) into slot r & 1.
    unsigned ph_val[2];
    float ph_mt[2], ph_md[2], ph_ist[2], ph_isd[2];
    int ph_tag[2];
    // Data wave -> control wave: the parked chunk's residual mass (tag: round).
    double rs_val[kDataWaves];
    int rs_tag[kDataWaves];
    // Set once a bounded wait expired: every later wait returns at once.
    int abort_wait;
    // End of the loop: deferred draws of this workgroup and the one at hand.
    int ntasks;
    int tk_draw;                                 // 1: scan tk_chunk
    int tk_chunk, tk_mode;                       // mode: 0 target row, 1 residual
    double tk_thr;
    float tk_mt, tk_md, tk_ist, tk_isd;
    // Block-wide scan scratch (deferred draws only, under barriers).
    double scan_ws[kMaxSub * kDataWaves];
    double red_d[kWaves];
    float red_f[kWaves];
    int red_i[kWaves];
    int sub_star;
    double sub_base;
};

// Relaxed workgroup-scope accesses for the mailboxes.
__device__ __forceinline__ void lds_put(int* p, int v) {
    __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
}
__device__ __forceinline__ int lds_get(int* p) {
    return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
}
// Compiler-only ordering point between a payload and its tag.
__device__ __forceinline__ void order() { __atomic_signal_fence(__ATOMIC_SEQ_CST); }

// Record a synchronisation time-out: the status word gets the flag, later
// waits of the workgroup return at once, and the kernel runs to its end with
// outputs that are not valid.
__device__ __forceinline__ void give_up(const Params& P, Shared& sh) {
    atomicOr(P.status, SV_FLAG_SYNC_TIMEOUT);
    lds_put(&sh.abort_wait, 1);
}

// Poll an LDS tag until it equals want (bounded).
__device__ __forceinline__ void lds_wait(const Params& P, Shared& sh, int* tag, int want) {
    for (unsigned it = 0; lds_get(tag) != want; ++it) {
        if (it >= kLdsSpinLimit || lds_get(&sh.abort_wait)) {
            give_up(P, sh);
            break;
        }
        __builtin_amdgcn_s_sleep(1);
    }
    order();
}

// ------------------------------------------------------ wave reductions --

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

__device__ __forceinline__ unsigned long long* dec_word(const Params& P, int tr) {
    return reinterpret_cast<unsigned long long*>(P.team + (size_t)tr * kTeamWords + TW_DEC);
}

// Control lane: team tr = (b, i) of a request with budget k is complete (its
// decision and, if it drew one, its token are stored). The team completing
// last for request b writes the request's outputs: j = the first rejected
// position (k if none), the token drawn by team j.
template <bool kGreedy>
__device__ void team_complete(const Params& P, int b, int k) {
    drain();
    const unsigned old = add32(&P.req_count[b * kReqStride], 1u);
    if (old != (unsigned)k) return;
    const int K = P.K;
    const int tr0 = b * (K + 1);
    int j = k;
    for (int t = 0; t < k; ++t) {
        if ((ld64(dec_word(P, tr0 + t)) & 1ull) == 0) {
            j = t;
            break;
        }
    }
    const int y = (int)ld32(&P.result[tr0 + j]);
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
    // Every unit of the request has been counted: reset the counters for the
    // next call (tagged words carry the call epoch and need no reset).
    if (kGreedy) {
        for (int t = 0; t <= k; ++t) st32(P.team + (size_t)(tr0 + t) * kTeamWords + TW_ARRIVE, 0u);
    }
    st32(&P.req_count[b * kReqStride], 0u);
}

// ------------------------------------------------------------ greedy leader --

// Control wave, greedy: merge the chunk argmaxes of target row i, decide,
// complete the team.
__device__ void leader_greedy(const Params& P, int b, int i, int k, int tr) {
    const int lane = threadIdx.x & 63;
    const int C = P.C;
    float bv = -INFINITY;
    int bi = INT_MAX;
    for (int cc = lane; cc < C; cc += 64) {
        const unsigned long long w = ld64(&P.rec[((size_t)tr * C + cc) * kRecWords]);
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
        }
        st32(&P.result[tr], (unsigned)best);
        st64(dec_word(P, tr), ((unsigned long long)P.epoch << 32) | (accept ? 1u : 0u));
        team_complete<true>(P, b, k);
    }
}

// ----------------------------------------------------- sampled team merge --

// Team-wide normalisers (identical in every workgroup that computes them:
// same inputs, same lanes, same reduction order).
struct TeamStats {
    float mt, md;      // max of the target / drafter row
    double st, sd;     // sum of 2^((z - max) c) over the row
};

// Control wave: wait until the C records of team tr are complete (bounded),
// then merge them: M = max of chunk maxima, S = sum of S_c 2^((M_c - M) c).
// Lane l holds chunks l, l + 64, l + 128 (C <= kMaxChunks).
__device__ TeamStats merge_team(const Params& P, Shared& sh, int tr) {
    const int lane = threadIdx.x & 63;
    const int C = P.C;
    const unsigned ep = P.epoch;
    unsigned long long* rec = P.rec + (size_t)tr * C * kRecWords;
    constexpr int Q = kMaxChunks / 64;
    unsigned long long w[Q][kStatWords];
    for (unsigned it = 0;; ++it) {
        bool ok = true;
        #pragma unroll
        for (int q = 0; q < Q; ++q) {
            const int cc = lane + 64 * q;
            #pragma unroll
            for (int f = 0; f < kStatWords; ++f) {
                w[q][f] = cc < C ? ld64(rec + cc * kRecWords + f) : (unsigned long long)ep;
            }
        }
        #pragma unroll
        for (int q = 0; q < Q; ++q) {
            #pragma unroll
            for (int f = 0; f < kStatWords; ++f) ok = ok && tag_ok(w[q][f], ep);
        }
        if (__ballot(!ok) == 0) break;
        if (it >= kSpinLimit || lds_get(&sh.abort_wait)) {
            if (lane == 0) give_up(P, sh);
            break;
        }
        __builtin_amdgcn_s_sleep(1);
    }
    float mt = -INFINITY, md = -INFINITY;
    #pragma unroll
    for (int q = 0; q < Q; ++q) {
        if (lane + 64 * q < C) {
            mt = fmaxf(mt, tag_val(w[q][R_MT]));
            md = fmaxf(md, tag_val(w[q][R_MD]));
        }
    }
    mt = wave_max(mt);
    md = wave_max(md);
    double st = 0.0, sd = 0.0;
    #pragma unroll
    for (int q = 0; q < Q; ++q) {
        if (lane + 64 * q < C) {
            const float s1 = tag_val(w[q][R_ST]), s2 = tag_val(w[q][R_SD]);
            if (s1 > 0.0f) st += (double)s1 * exp2(((double)tag_val(w[q][R_MT]) - (double)mt) * P.c64);
            if (s2 > 0.0f) sd += (double)s2 * exp2(((double)tag_val(w[q][R_MD]) - (double)md) * P.c64);
        }
    }
    TeamStats t;
    t.mt = mt;
    t.md = md;
    t.st = wave_sum(st);
    t.sd = wave_sum(sd);
    return t;
}

// Control wave: queue a deferred draw (team tr; bonus or rejection).
__device__ __forceinline__ void add_task(const Params& P, int tr, bool bonus, int& ntasks) {
    if ((threadIdx.x & 63) == 0 && ntasks < P.task_cap) {
        st32(reinterpret_cast<unsigned*>(P.tasks) + (size_t)blockIdx.x * P.task_cap + ntasks,
             (unsigned)(2 * tr + (bonus ? 1 : 0)));
    }
    ++ntasks;
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

// Control wave: collect the data waves' statistics of the unit of round r,
// merge them and publish the unit's record. Greedy: count the arrival and
// lead the team if last. Sampled: queue the bonus draw from the chunk-0
// member of a bonus position.
template <typename E, bool kGreedy>
__device__ __forceinline__ void control_unit(const Params& P, Shared& sh, const Unit& cur, int r,
                                             int& ntasks) {
    const int lane = threadIdx.x & 63;
    const int C = P.C;
    const int slot = r & 1;
    if (lane < kDataWaves) lds_wait(P, sh, &sh.st_tag[slot][lane], r + 1);
    unsigned long long* rec = P.rec + ((size_t)cur.tr * C + cur.c) * kRecWords;
    if (kGreedy) {
        float bv = -INFINITY;
        int bi = INT_MAX;
        if (lane < kDataWaves) {
            bv = sh.st_mt[slot][lane];
            bi = sh.st_idx[slot][lane];
        }
        order();
        if (lane == 0) lds_put(&sh.st_done[slot], r + 1);
        #pragma unroll
        for (int o = 32; o > 0; o >>= 1) {
            const float ov = __shfl_xor(bv, o, 64);
            const int oi = __shfl_xor(bi, o, 64);
            if (better_arg(ov, oi, bv, bi)) {
                bv = ov;
                bi = oi;
            }
        }
        int lead = 0;
        if (lane == 0) {
            st64(rec, ((unsigned long long)__float_as_uint(bv) << 32) | (unsigned)bi);
            drain();
            const unsigned old = add32(&P.team[(size_t)cur.tr * kTeamWords + TW_ARRIVE], 1u);
            lead = old == (unsigned)C - 1;
        }
        lead = __shfl(lead, 0, 64);
        if (lead) leader_greedy(P, cur.b, cur.i, cur.k, cur.tr);
    } else {
        float mt = -INFINITY, md = -INFINITY;
        double a = 0.0, d = 0.0;
        if (lane < kDataWaves) {
            mt = sh.st_mt[slot][lane];
            md = sh.st_md[slot][lane];
            a = sh.st_st[slot][lane];
            d = sh.st_sd[slot][lane];
        }
        order();
        if (lane == 0) lds_put(&sh.st_done[slot], r + 1);
        const float Mt = wave_max(mt), Md = wave_max(md);
        // Rescale each wave's sum from its own maximum to the chunk maximum.
        if (a > 0.0) a *= (double)fast_exp2((mt - Mt) * P.c32);
        if (d > 0.0) d *= (double)fast_exp2((md - Md) * P.c32);
        const double St = wave_sum(a), Sd = wave_sum(d);
        if (lane == 0) {
            const unsigned ep = P.epoch;
            st64(rec + R_MT, tagged(Mt, ep));
            st64(rec + R_MD, tagged(Md, ep));
            st64(rec + R_ST, tagged((float)St, ep));
            st64(rec + R_SD, tagged((float)Sd, ep));
        }
        if (cur.i == cur.k && cur.c == 0) add_task(P, cur.tr, true, ntasks);
    }
}

// Control wave, sampled: the parked unit of round r - 1 (drafted position i
// of request b, drafted token x loaded a round earlier). Wait for its team's
// records, take the team's decision, post it to the data waves; on a
// rejection that may be the request's first, collect and publish the chunk's
// residual mass. The chunk-0 member also writes p(x), q(x) and the decision
// word, and completes the team or queues its draw.
template <typename E>
__device__ __forceinline__ void control_parked(const Params& P, Shared& sh, const Unit& prev, int x,
                                               int r, int& ntasks) {
    const int lane = threadIdx.x & 63;
    const int K = P.K;
    const int slot = r & 1;
    const unsigned ep = P.epoch;
    const E* target = static_cast<const E*>(P.target);
    const E* draft = static_cast<const E*>(P.draft);
    // Issued before the records are awaited: the drafted token's logits and
    // the decisions of the request's earlier positions known so far.
    const bool valid = x >= 0 && x < P.V;
    float zt = 0.0f, zd = 0.0f;
    if (valid) {
        zt = Elem<E>::one(target + ((size_t)prev.b * (K + 1) + prev.i) * (size_t)P.V + x);
        zd = Elem<E>::one(draft + ((size_t)prev.b * K + prev.i) * (size_t)P.V + x);
    }
    unsigned long long dprev = 0;
    if (lane < prev.i) dprev = ld64(dec_word(P, prev.b * (K + 1) + lane));
    const TeamStats ts = merge_team(P, sh, prev.tr);
    double px = 0.0, qx = 0.0;
    if (valid) {
        px = exp2(((double)zt - (double)ts.mt) * P.c64) / ts.st;
        qx = exp2(((double)zd - (double)ts.md) * P.c64) / ts.sd;
    }
    const uint4 rw = philox4x32_10((uint32_t)prev.b, (uint32_t)prev.i, 0u, 0u, P.key0, P.key1);
    const bool accept = word_to_uniform(rw.x) * qx < px;
    // An earlier position already known to be rejected: no draw will be
    // needed for this one, whatever its decision.
    const bool later = __ballot(lane < prev.i && (unsigned)(dprev >> 32) == ep &&
                                (dprev & 1ull) == 0) != 0;
    const bool residual = !accept && !later;
    const float ist = (float)(1.0 / ts.st), isd = (float)(1.0 / ts.sd);
    if (lane == 0) {
        sh.ph_val[slot] = residual ? PH_REJECT : PH_ACCEPT;
        sh.ph_mt[slot] = ts.mt;
        sh.ph_md[slot] = ts.md;
        sh.ph_ist[slot] = ist;
        sh.ph_isd[slot] = isd;
        order();
        lds_put(&sh.ph_tag[slot], r);
    }
    const bool books = prev.c == 0;
    if (books && lane == 0) {
        if (!valid) atomicOr(P.status, SV_FLAG_BAD_TOKEN);
        if (P.out_p) P.out_p[(size_t)prev.b * K + prev.i] = (float)px;
        if (P.out_q) P.out_q[(size_t)prev.b * K + prev.i] = (float)qx;
        st64(dec_word(P, prev.tr), ((unsigned long long)ep << 32) | (accept ? 1u : 0u));
        if (!residual) team_complete<false>(P, prev.b, prev.k);
    }
    if (!residual) return;
    if (books) add_task(P, prev.tr, false, ntasks);
    // Residual mass of the parked chunk: one partial per data wave.
    double v = 0.0;
    if (lane < kDataWaves) {
        lds_wait(P, sh, &sh.rs_tag[lane], r);
        v = sh.rs_val[lane];
    }
    v = wave_sum(v);
    if (lane == 0) {
        st64(P.rec + ((size_t)prev.tr * P.C + prev.c) * kRecWords + R_RES,
             tagged((float)v, ep));
    }
}

// The control wave's loop. Round r: the parked unit of round r - 1 (its
// team's decision, started as soon as that unit is published), then the unit
// of round r (publish).
template <typename E, bool kGreedy, bool kVec>
__device__ __forceinline__ int control_loop(const Params& P, Shared& sh, const int* off) {
    const int U = off[P.B];
    const int G = gridDim.x;
    Unit cur = decode_unit(P, off, blockIdx.x, U, kGreedy);
    Unit prev;
    prev.u = -1;
    int x_prev = 0;
    int ntasks = 0;
    for (int r = 0; cur.u >= 0 || prev.u >= 0; ++r) {
        if (!kGreedy && prev.u >= 0) control_parked<E>(P, sh, prev, x_prev, r, ntasks);
        prev.u = -1;
        if (cur.u >= 0) {
            control_unit<E, kGreedy>(P, sh, cur, r, ntasks);
            if (cur.has_d) {
                prev = cur;
                x_prev = P.tokens[(size_t)cur.b * P.K + cur.i];   // used next round
            }
            cur = decode_unit(P, off, cur.u + G, U, kGreedy);
        }
    }
    return ntasks;
}

// The data waves' loop: stream units through registers, post per-wave
// statistics, park drafted units in LDS until their team has decided.
template <typename E, bool kGreedy, bool kVec>
__device__ __forceinline__ void data_loop(const Params& P, Shared& sh, const int* off,
                                          uint4* stash) {
    constexpr int W = Elem<E>::W;
    const int lane = threadIdx.x & 63;
    const int dw = (threadIdx.x >> 6) - 1;         // data wave index
    const int dt = threadIdx.x - 64;               // data thread index
    const int U = off[P.B];
    const int G = gridDim.x;
    const float cs = P.c32;

    uint4 gt[kG], gd[kG];
    Unit cur = decode_unit(P, off, blockIdx.x, U, kGreedy);
    if (cur.u >= 0) issue_loads<E, kVec>(P, cur, dt, gt, gd);
    bool have_prev = false;
    int r = 0;

    // The parked unit of round rr - 1: wait for its team's decision; on a
    // rejection, post this wave's part of the chunk's residual mass.
    auto finish_parked = [&](int rr) {
        const int slot = rr & 1;
        lds_wait(P, sh, &sh.ph_tag[slot], rr);
        if (sh.ph_val[slot] != PH_REJECT) return;
        const float mt = sh.ph_mt[slot], md = sh.ph_md[slot];
        const float ist = sh.ph_ist[slot], isd = sh.ph_isd[slot];
        float lr = 0.0f;
        #pragma unroll 1
        for (int j = 0; j < kG; ++j) {
            // Each lane reads back only the groups it parked itself.
            const uint4 a = stash[(0 * kG + j) * kDataThreads + dt];
            const uint4 d = stash[(1 * kG + j) * kDataThreads + dt];
            float m8[W];
            #pragma unroll
            for (int kk = 0; kk < W; ++kk) {
                const float pv = fast_exp2((Elem<E>::at(a, kk) - mt) * cs) * ist;
                const float qv = fast_exp2((Elem<E>::at(d, kk) - md) * cs) * isd;
                m8[kk] = fmaxf(0.0f, pv - qv);
            }
            #pragma unroll
            for (int h = W / 2; h > 0; h >>= 1) {
                #pragma unroll
                for (int kk = 0; kk < h; ++kk) m8[kk] += m8[kk + h];
            }
            lr += m8[0];
        }
        const double v = wave_sum((double)lr);
        if (lane == 0) {
            sh.rs_val[dw] = v;
            order();
            lds_put(&sh.rs_tag[dw], rr);
        }
    };

    for (; cur.u >= 0; ++r) {
        const int slot = r & 1;
        // Per-wave statistics of the unit of round r.
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
                if (r >= 2) lds_wait(P, sh, &sh.st_done[slot], r - 1);
                sh.st_mt[slot][dw] = bv;
                sh.st_idx[slot][dw] = bi;
                order();
                lds_put(&sh.st_tag[slot][dw], r + 1);
            }
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
            // than keeping every converted float alive across the reduction.
            #pragma unroll
            for (int j = 0; j < kG; ++j) {
                asm volatile("" : "+v"(gt[j].x), "+v"(gt[j].y), "+v"(gt[j].z), "+v"(gt[j].w));
                asm volatile("" : "+v"(gd[j].x), "+v"(gd[j].y), "+v"(gd[j].z), "+v"(gd[j].w));
            }
            mt = wave_max(mt);
            md = wave_max(md);
            float lt = 0.0f, ld = 0.0f;
            if (mt != -INFINITY) {
                #pragma unroll
                for (int j = 0; j < kG; ++j) {
                    float e[W];
                    #pragma unroll
                    for (int kk = 0; kk < W; ++kk) e[kk] = fast_exp2((Elem<E>::at(gt[j], kk) - mt) * cs);
                    #pragma unroll
                    for (int h = W / 2; h > 0; h >>= 1) {
                        #pragma unroll
                        for (int kk = 0; kk < h; ++kk) e[kk] += e[kk + h];
                    }
                    lt += e[0];
                }
            }
            if (cur.has_d && md != -INFINITY) {
                #pragma unroll
                for (int j = 0; j < kG; ++j) {
                    float e[W];
                    #pragma unroll
                    for (int kk = 0; kk < W; ++kk) e[kk] = fast_exp2((Elem<E>::at(gd[j], kk) - md) * cs);
                    #pragma unroll
                    for (int h = W / 2; h > 0; h >>= 1) {
                        #pragma unroll
                        for (int kk = 0; kk < h; ++kk) e[kk] += e[kk + h];
                    }
                    ld += e[0];
                }
            }
            const double st = wave_sum((double)lt);
            const double sd = wave_sum((double)ld);
            if (lane == 0) {
                if (r >= 2) lds_wait(P, sh, &sh.st_done[slot], r - 1);
                sh.st_mt[slot][dw] = mt;
                sh.st_md[slot][dw] = md;
                sh.st_st[slot][dw] = st;
                sh.st_sd[slot][dw] = sd;
                order();
                lds_put(&sh.st_tag[slot][dw], r + 1);
            }
        }

        // The stash is free once the previous parked unit is done with.
        if (have_prev) finish_parked(r);

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
        have_prev = cur.has_d;
        cur = nxt;
    }
    if (have_prev) finish_parked(r);
}

// Control wave: prepare deferred draw number t of this workgroup (team
// b, i): wait until the earlier positions of the request are decided; draw
// only if none of them rejected (i is the request's first rejection, or the
// bonus position with no rejection). Locate the chunk that holds the
// threshold and leave its element scan to the whole workgroup.
__device__ void task_prepare(const Params& P, Shared& sh, int task) {
    const int lane = threadIdx.x & 63;
    const int K = P.K, C = P.C;
    const unsigned ep = P.epoch;
    const int tr = task >> 1;
    const bool bonus = task & 1;
    const int b = tr / (K + 1), i = tr - b * (K + 1);
    // Earlier positions (lane t polls position t): done once every position
    // before the first known rejection is decided, or all are decided.
    bool first = true;
    for (unsigned it = 0;; ++it) {
        unsigned long long d = 0;
        if (lane < i) d = ld64(dec_word(P, b * (K + 1) + lane));
        const bool known = lane >= i || (unsigned)(d >> 32) == ep;
        const unsigned long long rej = __ballot(lane < i && known && (d & 1ull) == 0);
        const unsigned long long unknown = __ballot(!known);
        if (rej != 0) {
            const unsigned long long below = (rej & (~rej + 1)) - 1;   // lanes below the first rejection
            if ((unknown & below) == 0) {
                first = false;
                break;
            }
        } else if (unknown == 0) {
            break;
        }
        if (it >= kSpinLimit || lds_get(&sh.abort_wait)) {
            if (lane == 0) give_up(P, sh);
            first = false;
            break;
        }
        __builtin_amdgcn_s_sleep(2);
    }
    int draw = 0, chunk = -1, mode = 0;
    double thr = 0.0;
    TeamStats ts;
    ts.mt = ts.md = 0.0f;
    ts.st = ts.sd = 1.0;
    if (first) {
        ts = merge_team(P, sh, tr);
        unsigned long long* rec = P.rec + (size_t)tr * C * kRecWords;
        const uint4 rw = philox4x32_10((uint32_t)b, (uint32_t)i, 0u, 0u, P.key0, P.key1);
        const double u = word_to_uniform(rw.y);
        double total = 0.0, base = 0.0;
        if (!bonus) {
            // Residual masses: all C members publish theirs.
            for (unsigned it = 0;; ++it) {
                bool ok = true;
                for (int cc = lane; cc < C; cc += 64) ok = ok && tag_ok(ld64(rec + cc * kRecWords + R_RES), ep);
                if (__ballot(!ok) == 0) break;
                if (it >= kSpinLimit || lds_get(&sh.abort_wait)) {
                    if (lane == 0) give_up(P, sh);
                    break;
                }
                __builtin_amdgcn_s_sleep(1);
            }
            auto rmass = [&](int cc) -> double {
                const float v = tag_val(ld64(rec + cc * kRecWords + R_RES));
                return v > 0.0f ? (double)v : 0.0;
            };
            for (int cc = lane; cc < C; cc += 64) total += rmass(cc);
            total = wave_sum(total);
            if (total > 0.0) {
                chunk_crossing(C, u * total, rmass, chunk, base);
                mode = 1;
            }
        }
        if (chunk < 0 && ts.st > 0.0) {
            // Bonus draw, or a residual without mass (rounding only): from p_i.
            mode = 0;
            const double inv = 1.0 / ts.st;
            auto pmass = [&](int cc) -> double {
                const float s1 = tag_val(ld64(rec + cc * kRecWords + R_ST));
                const float m1 = tag_val(ld64(rec + cc * kRecWords + R_MT));
                return s1 > 0.0f ? (double)s1 * exp2(((double)m1 - (double)ts.mt) * P.c64) * inv : 0.0;
            };
            total = 0.0;
            for (int cc = lane; cc < C; cc += 64) total += pmass(cc);
            total = wave_sum(total);
            chunk_crossing(C, u * total, pmass, chunk, base);
        }
        draw = 1;
        thr = u * total - base;
    }
    if (lane == 0) {
        sh.tk_draw = draw;
        sh.tk_chunk = chunk;
        sh.tk_mode = mode;
        sh.tk_thr = thr;
        sh.tk_mt = ts.mt;
        sh.tk_md = ts.md;
        sh.tk_ist = (float)(1.0 / ts.st);
        sh.tk_isd = (float)(1.0 / ts.sd);
    }
}

// Deferred draws of this workgroup (whole workgroup, under barriers).
template <typename E, bool kVec>
__device__ __forceinline__ void run_tasks(const Params& P, Shared& sh) {
    const int K = P.K;
    const int nt = min(sh.ntasks, P.task_cap);
    const E* target = static_cast<const E*>(P.target);
    const E* draft = static_cast<const E*>(P.draft);
    unsigned* list = reinterpret_cast<unsigned*>(P.tasks) + (size_t)blockIdx.x * P.task_cap;
    for (int t = 0; t < nt; ++t) {
        const int task = (int)ld32(list + t);
        if (threadIdx.x < 64) task_prepare(P, sh, task);
        __syncthreads();
        const int tr = task >> 1;
        const int b = tr / (K + 1), i = tr - b * (K + 1);
        int y = 0;
        if (sh.tk_draw && sh.tk_chunk >= 0) {
            const int e0 = sh.tk_chunk * P.CE;
            const int n = min(P.CE, P.V - e0);
            const E* rt = target + ((size_t)b * (K + 1) + i) * (size_t)P.V + e0;
            const E* rd = sh.tk_mode == 1 ? draft + ((size_t)b * K + i) * (size_t)P.V + e0 : nullptr;
            const int o = chunk_scan<E, kVec>(sh, rt, rd, n, sh.tk_mt, sh.tk_ist, sh.tk_md,
                                              sh.tk_isd, P.c32, sh.tk_thr);
            y = o < 0 ? 0 : e0 + o;
        }
        if (threadIdx.x == 0) {
            // The request's budget, clamped as in the prologue.
            int k = P.budgets[b];
            k = k < 0 ? 0 : (k > K ? K : k);
            if (sh.tk_draw) st32(&P.result[tr], (unsigned)y);
            team_complete<false>(P, b, k);
        }
        __syncthreads();
    }
}

template <typename E, bool kGreedy, bool kVec>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(4)))
void verify_kernel(Params P) {
    extern __shared__ __align__(16) unsigned char dyn_smem[];
    __shared__ Shared sh;
    // Dynamic LDS: the parked unit (sampled mode), then request unit offsets.
    uint4* stash = reinterpret_cast<uint4*>(dyn_smem);
    int* off = reinterpret_cast<int*>(dyn_smem + (kGreedy ? 0 : (size_t)2 * kG * kDataThreads * 16));

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int B = P.B, K = P.K, C = P.C;

    // Prologue: every workgroup scans the budgets into per-request unit
    // offsets, and clears the mailbox tags.
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
        if (tid < 2 * kDataWaves) (&sh.st_tag[0][0])[tid] = 0;
        if (tid < kDataWaves) sh.rs_tag[tid] = -1;
        if (tid < 2) {
            sh.ph_tag[tid] = -1;
            sh.st_done[tid] = 0;
        }
        if (tid == 0) sh.abort_wait = 0;
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
        __syncthreads();
    }

    // Wave specialisation (the branch is uniform per wave). No barrier
    // until both loops are done.
    if (__builtin_amdgcn_readfirstlane(wave) == 0) {
        const int nt = control_loop<E, kGreedy, kVec>(P, sh, off);
        if (lane == 0) sh.ntasks = nt;
        drain();                                   // task list entries are written
    } else {
        data_loop<E, kGreedy, kVec>(P, sh, off, stash);
    }
    __syncthreads();
    if (!kGreedy) run_tasks<E, kVec>(P, sh);
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
    unsigned long long* rec;
    unsigned* team;
    unsigned* result;
    unsigned* req_count;
    unsigned* status;
    int* tasks;
    size_t task_words;             // entries of the task lists' region
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
    // Task lists: at most two deferred draws per round of a workgroup.
    const long long units = (long long)p.B * (p.K + 1) * p.C;
    const long long cap = 2 * ((units + grid - 1) / grid) + 2;
    if (cap > INT_MAX || (size_t)(grid * cap) > ctx->task_words) return SV_ERR_ARG;
    p.tasks = ctx->tasks;
    p.task_cap = (int)cap;
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
    if (chunks_for(vocab, dtype) > kMaxChunks) return SV_ERR_ARG;   // not reachable for legal V
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
    const size_t rec_bytes = round256(teams * c->C * kRecWords * 8);
    const size_t team_bytes = round256(teams * kTeamWords * 4);
    const size_t result_bytes = round256(teams * 4);
    const size_t req_bytes = round256((size_t)max_batch * kReqStride * 4);
    // Task lists: 2 entries per unit plus 4 per workgroup bound every launch
    // (at most 4 resident workgroups per CU of 8 waves; 16 allowed for).
    c->task_words = 2 * teams * (size_t)c->C + 4 * (size_t)c->cus * 16;
    const size_t task_bytes = round256(c->task_words * 4);
    const size_t total = rec_bytes + team_bytes + result_bytes + req_bytes + task_bytes + 256;
    if (rc == SV_OK && hipMalloc(&c->ws, total) != hipSuccess) {
        c->ws = nullptr;
        rc = SV_ERR_NOMEM;
    }
    if (rc == SV_OK) {
        unsigned char* w = static_cast<unsigned char*>(c->ws);
        size_t o = 0;
        c->rec = reinterpret_cast<unsigned long long*>(w + o);
        o += rec_bytes;
        c->team = reinterpret_cast<unsigned*>(w + o);
        o += team_bytes;
        c->result = reinterpret_cast<unsigned*>(w + o);
        o += result_bytes;
        c->req_count = reinterpret_cast<unsigned*>(w + o);
        o += req_bytes;
        c->tasks = reinterpret_cast<int*>(w + o);
        o += task_bytes;
        c->status = reinterpret_cast<unsigned*>(w + o);
        if (hipMemset(c->ws, 0, total) != hipSuccess || hipDeviceSynchronize() != hipSuccess) {
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
    p.rec = ctx->rec;
    p.team = ctx->team;
    p.result = ctx->result;
    p.req_count = ctx->req_count;
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
    ctx->calls = ctx->calls % 0xFFFFFFFFu + 1u;     // 1 .. 2^32 - 1, never 0
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
