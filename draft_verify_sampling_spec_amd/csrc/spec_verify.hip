// spec_verify.hip -- batched draft verification for MI355X (gfx950, wave64).
//
// What is computed: "Speculative decoding becomes standard: DSpark and
// multi-token drafters", section "Why draft-and-verify does not change the
// output" (greedy keep-while-agreeing rule, paragraph 1; the sampled
// min(1, p/q) acceptance with residual resampling, paragraph 2), with the
// per-request verify budgets of section "What DSpark adds", paragraph 2.
// The ABI and its conventions are documented in include/spec_verify.h.
//
// Design: a streaming pass reads every logit row the method needs exactly
// once (and takes the greedy decisions); in sampled mode a draw pass follows
// on the stream, decides the drafted positions and makes each request's one
// draw.
//  * Work unit = vocabulary chunk c of position i of request b: the chunk of
//    target row i and, for a drafted position, the same chunk of drafter row
//    i. Every chunk of a call has the same size: 960 data lanes x 4
//    sixteen-byte loads per row when sampled, x 8 when greedy (one row per
//    unit, so the same bytes in flight). Units are numbered request-major,
//    position-major, chunk-minor, so the C chunks of one position (a "team")
//    are consecutive.
//  * Streaming pass (verify_kernel): one workgroup of 16 waves per CU, grid =
//    the resident workgroups. Units are handed out dynamically: the first
//    rounds of workgroup w take units w, w + G, ..., later ones the values of
//    a device-scope counter, so faster workgroups take more units and the C
//    units of a team are taken, and finish, close together. Waves 1-15
//    stream data: 16-byte loads of a unit into registers, reduced per wave to
//    the scaled max s = max(z) c and the sum of 2^(z c - s), c = log2(e)/T
//    (sampled; one fused multiply-add and an exp2 per element), or (max,
//    lowest index) (greedy), posted to LDS; the next unit's loads go out
//    group by group as the reduction consumes the registers. They never wait
//    on another workgroup. Wave 0 is the control wave: it plans the units a
//    few rounds ahead, merges the waves' statistics and publishes the chunk's
//    record; the two kinds of waves exchange tagged LDS messages, with no
//    workgroup barrier in the loop.
//  * Greedy: the control wave posts the chunk's (max, first index) as a
//    64-bit key to its team's atomic maximum, then counts the unit on its
//    request's counter; the workgroup that counts a request's last unit
//    reads the request's team keys (each a row's first argmax), decides and
//    writes the outputs. Sampled: every record word carries the call's
//    epoch, and the chunk of a drafted position that holds the drafted
//    token adds that token's two logits to its record.
//  * Draw pass (draw_kernel, sampled): one 8-wave workgroup per request, two
//    per CU. Its waves decide the request's drafted positions side by side
//    (p(x) and q(x) from each team's records, the accept test), then it
//    streams the first rejected position's target and drafter rows once for
//    the residual masses of 512-element blocks and scans the block holding
//    the threshold; the bonus position picks its chunk from the records' p
//    masses and streams that chunk's blocks the same way. It writes the
//    request's outputs. Nothing in it waits on another workgroup.
//  * No wave of either pass waits on another workgroup, so neither pass
//    depends on which of its workgroups are resident at a time: a greedy
//    team is decided by whichever workgroup completes it, and each launch
//    clears the schedule counter of the launch after it.
//  * Synchronisation uses device-scope relaxed atomics (plus s_waitcnt where
//    a counter orders earlier stores), never release/acquire fences: those
//    write back and invalidate the whole L2.

#include <hip/hip_runtime.h>

#include <climits>
#include <cmath>
#include <cstdint>
#include <cstring>
#include <mutex>
#include <type_traits>
#include <vector>

#include "philox_device.h"
#include "spec_verify.h"

namespace {

// The wave count is a multiple of 4 so that every SIMD holds the same number
// of a workgroup's waves (with 5 waves, the hardware reserves two wave slots
// per SIMD per workgroup and fewer workgroups fit than the occupancy query
// reports).
constexpr int kWaves = 16;                     // wave 0: control; waves 1-15: data
constexpr int kThreads = kWaves * 64;
constexpr int kDataWaves = kWaves - 1;
constexpr int kDataThreads = kDataWaves * 64;
constexpr int kG = 4;                          // 16-byte groups per data lane per row of a sampled unit
constexpr int kLaunchBatch = 8192;             // requests per launch (unit offsets live in LDS)
constexpr int kMbox = 1;                       // result mailbox slots (rounds the data waves may lead)
constexpr int kPlanLead = 4;                   // rounds the control wave plans ahead (>= kMbox)
constexpr int kPlanSlots = 8;                  // plan ring (> kPlanLead + 1)
static_assert(kPlanLead >= kMbox && kPlanSlots > kPlanLead + 1, "plan ring too short");
constexpr int PL_END = 0, PL_UNIT = 1;
constexpr int kBlocks = kG * kDataWaves;       // 64-group blocks (one 16-byte load per lane) in a chunk
// A greedy unit reads one row, so it takes twice the groups per lane: the
// same bytes in flight as a sampled unit of a drafted position.
template <bool kGreedy>
__host__ __device__ constexpr int groups_of() { return kGreedy ? 2 * kG : kG; }
constexpr int kTeamWords = 32;                 // words per team record (128 bytes)
constexpr int kReqStride = 16;                 // words between request counters (64 bytes)
constexpr unsigned kLdsSpinLimit = 1u << 26;   // bounded LDS mailbox wait (~3 s)

// Team record words (greedy): a 64-bit argmax key, the atomic maximum of the
// team's chunk keys (arg_key), zero when no chunk has posted one.
constexpr int TW_KEY = 0;

// Scheduling words (Params::sched, 64 bytes apart): two counters of the next
// unit to hand out. A launch uses the one its epoch's parity names, and
// clears the other, which the launch before it used (launches on one
// workspace are stream-ordered and their epochs alternate in parity), for
// the launch after it. So no workgroup has to find out that it finished
// last in order to reset the schedule.
constexpr int SC_NEXT0 = 0, SC_NEXT1 = 16;

// Unit record: 6 64-bit words.
//   sampled: word f = (value bits << 32) | epoch for the fp32 values
//            R_MT the scaled maximum s_t = max(z_t) c (c = log2(e) / T,
//            rounded once), R_MD likewise for z_d, R_ST the sum of
//            2^(z_t c - s_t), R_SD likewise
//            and, in the one chunk of a drafted position that holds its
//            drafted token x, R_ZT = (z_t(x) bits << 32) | epoch, R_ZD
//            likewise for z_d(x)
//   greedy:  word R_MT = (max bits << 32) | epoch, word R_MD = (lowest index
//            of the max << 32) | epoch
constexpr int kRecWords = 6;
constexpr int R_MT = 0, R_MD = 1, R_ST = 2, R_SD = 3, R_ZT = 4, R_ZD = 5;
constexpr int kStatWords = 4;   // words R_MT..R_SD make a record complete

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
    unsigned* team;                // [B*(K+1)][kTeamWords]: greedy argmax keys
    unsigned* req_count;           // [B][kReqStride]: greedy: units counted
    unsigned* sched;               // scheduling words SC_NEXT0, SC_NEXT1
    unsigned* status;              // 1 word
    double* dmass;                 // draw pass split over workgroups: block masses [requests][C * kBlocks]
    unsigned* dcnt;                // draw pass split: slices finished per request, kReqStride apart
    int dsplit;                    // workgroups per request in the draw pass
    int B, K, V;
    uint32_t bbase;                // Philox request index of request 0 of this launch
    int C;                         // chunks per row
    int CE;                        // elements per chunk
    float c32;                     // log2(e) / T
    double c64;
    uint32_t key0, key1;
    unsigned epoch;                // call number (never 0): tags the sampled records
};

// The schedule counter of this launch.
__device__ __forceinline__ unsigned* sched_next(const Params& P) {
    return P.sched + ((P.epoch & 1u) ? SC_NEXT1 : SC_NEXT0);
}

// ------------------------------------------------------------- atomics --

__device__ __forceinline__ void st32(unsigned* p, unsigned v) {
    __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
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
__device__ __forceinline__ void max64(unsigned long long* p, unsigned long long v) {
    (void)__hip_atomic_fetch_max(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
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

using svrng::philox4x32_10;
using svrng::word_to_uniform;

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
    // Control wave -> data waves: the plan of data round q, written kPlanLead
    // rounds ahead into slot q % kPlanSlots: the next unit of the workgroup's
    // sequence, or the end of the loop.
    int pl_tag[kPlanSlots];
    int pl_kind[kPlanSlots];
    int pl_u[kPlanSlots], pl_b[kPlanSlots];      // unit and its request
    // Data wave -> control wave: a round's per-wave results, in slot
    // round % kMbox. Sampled: (scaled max s, sum of 2^(z c - s)) of the
    // target and drafter parts; greedy: (max, lowest index of the max).
    float st_mt[kMbox][kDataWaves];
    float st_md[kMbox][kDataWaves];
    double st_st[kMbox][kDataWaves];
    double st_sd[kMbox][kDataWaves];
    int st_idx[kMbox][kDataWaves];
    int st_tag[kMbox][kDataWaves];                   // round + 1
    int st_done[kMbox];                          // control wave: round + 1 of the slot it read last
    // Set once a bounded wait expired: every later wait returns at once.
    int abort_wait;
    // Prologue scratch under barriers: per-wave partial sums.
    int red_i[kWaves];
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

// Whole-wave reductions on the VALU's data-parallel primitives (DPP): a
// butterfly inside each quad (lane xor 1, xor 2), the row's half mirror and
// mirror (the 8- and 16-lane groups), then two row broadcasts that carry
// rows 0-2's results up so that lane 63 holds the whole wave's; one read of
// lane 63 makes the result uniform. No LDS traffic and no cross-lane wait on
// memory, unlike permutes through the LDS crossbar. The reduction order is
// fixed, so every wave that reduces the same values gets the same result.
constexpr int kDppXor1 = 0xB1, kDppXor2 = 0x4E;          // quad_perm [1,0,3,2], [2,3,0,1]
constexpr int kDppHalfMirror = 0x141, kDppMirror = 0x140;
constexpr int kDppBcast15 = 0x142, kDppBcast31 = 0x143;

// Lane's DPP source value under control CTRL; lanes of rows outside ROWS
// keep `identity`.
template <int CTRL, int ROWS = 0xF>
__device__ __forceinline__ int dpp32(int v, int identity) {
    return __builtin_amdgcn_update_dpp(identity, v, CTRL, ROWS, 0xF, false);
}
template <int CTRL, int ROWS = 0xF>
__device__ __forceinline__ float dppf(float v, float identity) {
    return __int_as_float(dpp32<CTRL, ROWS>(__float_as_int(v), __float_as_int(identity)));
}
template <int CTRL, int ROWS = 0xF>
__device__ __forceinline__ double dppd(double v) {                // identity 0.0
    const long long b = __double_as_longlong(v);
    const int lo = dpp32<CTRL, ROWS>((int)(unsigned)(unsigned long long)b, 0);
    const int hi = dpp32<CTRL, ROWS>((int)(b >> 32), 0);
    return __longlong_as_double(((long long)hi << 32) | (long long)(unsigned)lo);
}

__device__ __forceinline__ float lane63f(float v) {
    return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 63));
}
__device__ __forceinline__ double lane63d(double v) {
    const long long b = __double_as_longlong(v);
    const int lo = __builtin_amdgcn_readlane((int)(unsigned)(unsigned long long)b, 63);
    const int hi = __builtin_amdgcn_readlane((int)(b >> 32), 63);
    return __longlong_as_double(((long long)hi << 32) | (long long)(unsigned)lo);
}

__device__ __forceinline__ float wave_max(float v) {
    const float ni = -INFINITY;
    v = fmaxf(v, dppf<kDppXor1>(v, ni));
    v = fmaxf(v, dppf<kDppXor2>(v, ni));
    v = fmaxf(v, dppf<kDppHalfMirror>(v, ni));
    v = fmaxf(v, dppf<kDppMirror>(v, ni));
    v = fmaxf(v, dppf<kDppBcast15, 0xA>(v, ni));
    v = fmaxf(v, dppf<kDppBcast31, 0xC>(v, ni));
    return lane63f(v);
}

__device__ __forceinline__ double wave_sum(double v) {
    v += dppd<kDppXor1>(v);
    v += dppd<kDppXor2>(v);
    v += dppd<kDppHalfMirror>(v);
    v += dppd<kDppMirror>(v);
    v += dppd<kDppBcast15, 0xA>(v);
    v += dppd<kDppBcast31, 0xC>(v);
    return lane63d(v);
}

// The same reductions through the LDS crossbar (permutes). Waves whose
// bottleneck is the VALU (the streaming pass's data waves, the draw pass)
// use these: the permutes run on the otherwise idle LDS unit.
__device__ __forceinline__ double wave_sum_xbar(double v) {
    #pragma unroll
    for (int off = 32; off > 0; off >>= 1) v += __shfl_xor(v, off, 64);
    return v;
}
__device__ __forceinline__ float wave_max_xbar(float v) {
    #pragma unroll
    for (int off = 32; off > 0; off >>= 1) v = fmaxf(v, __shfl_xor(v, off, 64));
    return v;
}

__device__ __forceinline__ bool better_arg(float v, int i, float bv, int bi);

__device__ __forceinline__ void wave_argmax_xbar(float& bv, int& bi) {
    #pragma unroll
    for (int off = 32; off > 0; off >>= 1) {
        const float ov = __shfl_xor(bv, off, 64);
        const int oi = __shfl_xor(bi, off, 64);
        if (better_arg(ov, oi, bv, bi)) {
            bv = ov;
            bi = oi;
        }
    }
}

// (value, index) of the largest value, lowest index among equal values, over
// the wave (uniform result). Ties and the order of merging do not change it.
__device__ __forceinline__ void wave_argmax(float& bv, int& bi) {
    const float ni = -INFINITY;
#define SV_ARG_STEP(CTRL, ROWS)                                                 \
    {                                                                           \
        const float ov = dppf<CTRL, ROWS>(bv, ni);                              \
        const int oi = dpp32<CTRL, ROWS>(bi, INT_MAX);                          \
        if (better_arg(ov, oi, bv, bi)) {                                       \
            bv = ov;                                                            \
            bi = oi;                                                            \
        }                                                                       \
    }
    SV_ARG_STEP(kDppXor1, 0xF)
    SV_ARG_STEP(kDppXor2, 0xF)
    SV_ARG_STEP(kDppHalfMirror, 0xF)
    SV_ARG_STEP(kDppMirror, 0xF)
    SV_ARG_STEP(kDppBcast15, 0xA)
    SV_ARG_STEP(kDppBcast31, 0xC)
#undef SV_ARG_STEP
    bv = lane63f(bv);
    bi = __builtin_amdgcn_readlane(bi, 63);
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

// Wave 0: find the chunk where the running mass over chunks 0..C-1 first
// exceeds thr. mass(cc) gives chunk cc's mass. Returns (chunk, mass before it)
// in every lane; if rounding leaves no crossing, the last chunk with mass;
// chunk -1 if there is no mass.
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
    // No crossing (rounding): the last lane holding mass, whose last block
    // with mass is taken below.
    const unsigned long long pos = __ballot(acc > 0.0);
    const int lane_star = hit ? (__ffsll((long long)hit) - 1) : (pos ? 63 - __clzll((long long)pos) : 63);
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

// Greedy: the argmax key of (value v, index i). Larger keys have larger
// values, or equal values and lower indices, the order better_arg gives
// (-0 counts as +0; the merges never hand on a NaN); 0 is no key.
__device__ __forceinline__ unsigned long long arg_key(float v, int i) {
    const unsigned bits = __float_as_uint(v + 0.0f);
    const unsigned ord = (bits & 0x80000000u) ? ~bits : (bits | 0x80000000u);
    return ((unsigned long long)ord << 32) | (unsigned long long)(0xFFFFFFFFu - (unsigned)i);
}
__device__ __forceinline__ int key_index(unsigned long long key) {
    return key == 0ull ? 0 : (int)(0xFFFFFFFFu - (unsigned)key);   // no key: an all-NaN row, index 0
}
__device__ __forceinline__ unsigned long long* team_key(const Params& P, int tr) {
    return reinterpret_cast<unsigned long long*>(P.team + (size_t)tr * kTeamWords + TW_KEY);
}

// One lane: request b (budget k) ends at position j (the first rejection,
// k if none) with token y there: the accepted drafted tokens, y, then -1
// padding; probabilities past the positions the request decides are NaN
// (greedy decides none).
template <bool kGreedy>
__device__ void request_outputs(const Params& P, int b, int k, int j, int y) {
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
}

// Control wave, greedy: every unit of request b (budget k) has posted its
// chunk key and been counted. Read the k + 1 team keys (lane t: position t),
// take the decisions, write the outputs, and clear the keys and the counter
// for the next call.
__device__ void request_complete(const Params& P, int b, int k) {
    const int lane = threadIdx.x & 63;
    const int tr0 = b * (P.K + 1);
    unsigned long long key = 0ull;
    int x = -1;
    if (lane <= k) key = ld64(team_key(P, tr0 + lane));
    if (lane < k) x = P.tokens[(size_t)b * P.K + lane];
    const int best = key_index(key);
    const bool valid = x >= 0 && x < P.V;
    if (__ballot(lane < k && !valid) != 0ull && lane == 0) atomicOr(P.status, SV_FLAG_BAD_TOKEN);
    const unsigned long long rej = __ballot(lane < k && !(valid && x == best));
    const int j = rej != 0ull ? __builtin_ctzll(rej) : k;
    const int y = __shfl(best, j, 64);
    if (lane <= k) st64(team_key(P, tr0 + lane), 0ull);
    if (lane == 0) {
        request_outputs<true>(P, b, k, j, y);
        st32(&P.req_count[b * kReqStride], 0u);
    }
}

// ----------------------------------------------------------- team records --

// A team's C records as one control-wave load: lane l holds chunk l in
// registers; chunks 64 and up (vocabularies of more than 64 chunks) are read
// again where they are needed.
struct TeamPoll {
    unsigned long long w[kStatWords];
    int tr;
};

__device__ __forceinline__ unsigned long long* team_rec(const Params& P, int tr) {
    return P.rec + (size_t)tr * P.C * kRecWords;
}

__device__ __forceinline__ void poll_issue(const Params& P, int tr, TeamPoll& pl) {
    const int lane = threadIdx.x & 63;
    unsigned long long* rec = team_rec(P, tr);
    pl.tr = tr;
    #pragma unroll
    for (int f = 0; f < kStatWords; ++f) {
        pl.w[f] = lane < P.C ? ld64(rec + lane * kRecWords + f) : (unsigned long long)P.epoch;
    }
}

// True when every record word of the team carries this call's epoch.
__device__ __forceinline__ bool poll_complete(const Params& P, const TeamPoll& pl) {
    const int lane = threadIdx.x & 63;
    bool ok = true;
    #pragma unroll
    for (int f = 0; f < kStatWords; ++f) ok = ok && tag_ok(pl.w[f], P.epoch);
    if (P.C > 64) {
        unsigned long long* rec = team_rec(P, pl.tr);
        for (int cc = lane + 64; cc < P.C; cc += 64) {
            for (int f = 0; f < kStatWords; ++f) ok = ok && tag_ok(ld64(rec + cc * kRecWords + f), P.epoch);
        }
    }
    return __ballot(!ok) == 0;
}

// Team-wide normalisers (identical in every workgroup that computes them:
// same inputs, same lanes, same reduction order).
struct TeamStats {
    float mt, md;      // scaled maximum of the target / drafter row, max(z) c
    double st, sd;     // sum of 2^(z c - scaled maximum) over the row
};

// Merge complete sampled records: M = max of the chunks' scaled maxima,
// S = sum of S_c 2^(M_c - M).
__device__ TeamStats team_stats(const Params& P, const TeamPoll& pl) {
    const int lane = threadIdx.x & 63;
    const int C = P.C;
    unsigned long long* rec = team_rec(P, pl.tr);
    float mt = -INFINITY, md = -INFINITY;
    if (lane < C) {
        mt = tag_val(pl.w[R_MT]);
        md = tag_val(pl.w[R_MD]);
    }
    for (int cc = lane + 64; cc < C; cc += 64) {
        mt = fmaxf(mt, tag_val(ld64(rec + cc * kRecWords + R_MT)));
        md = fmaxf(md, tag_val(ld64(rec + cc * kRecWords + R_MD)));
    }
    mt = wave_max(mt);
    md = wave_max(md);
    double st = 0.0, sd = 0.0;
    auto add = [&](float m1, float m2, float s1, float s2) {
        if (s1 > 0.0f) st += (double)s1 * exp2((double)m1 - (double)mt);
        if (s2 > 0.0f) sd += (double)s2 * exp2((double)m2 - (double)md);
    };
    if (lane < C) add(tag_val(pl.w[R_MT]), tag_val(pl.w[R_MD]), tag_val(pl.w[R_ST]), tag_val(pl.w[R_SD]));
    for (int cc = lane + 64; cc < C; cc += 64) {
        add(tag_val(ld64(rec + cc * kRecWords + R_MT)), tag_val(ld64(rec + cc * kRecWords + R_MD)),
            tag_val(ld64(rec + cc * kRecWords + R_ST)), tag_val(ld64(rec + cc * kRecWords + R_SD)));
    }
    TeamStats t;
    t.mt = mt;
    t.md = md;
    t.st = wave_sum(st);
    t.sd = wave_sum(sd);
    return t;
}

// ---------------------------------------------------------- main kernel --

// Coordinates of a work unit (uniform across the workgroup).
struct Unit {
    int u;         // unit index, -1: none
    int b, i, k, c;
    int tr;        // team record index b * (K + 1) + i
    int e0, n;     // chunk start and length (elements)
    int n2;        // pair: length of chunk c + 1
    bool drafted;  // sampled, a drafted position: the drafter row's chunk c is read too
    bool pair;     // sampled, the bonus position: chunk c + 1 of the target row is read too
    bool has_d;    // drafted or pair: the second registers hold data
};

// Units of a request with budget k: greedy, C per position; sampled, C per
// drafted position and ceil(C / 2) for the bonus position, whose units take
// two consecutive chunks of its one row (the bytes in flight of a drafted
// unit).
__host__ __device__ __forceinline__ int bonus_units(int C, bool greedy) {
    return greedy ? C : (C + 1) >> 1;
}
__host__ __device__ __forceinline__ int request_units(int k, int C, bool greedy) {
    return k * C + bonus_units(C, greedy);
}

// The coordinates of unit u of request b (two independent LDS reads; no
// search). u < 0 gives the empty unit.
__device__ __forceinline__ Unit unit_from(const Params& P, const int* off, int u, int b, bool greedy) {
    Unit d;
    d.u = u;
    d.b = d.i = d.k = d.c = d.tr = d.e0 = d.n = d.n2 = 0;
    d.drafted = d.pair = d.has_d = false;
    if (u < 0) return d;
    d.b = b;
    const int C = P.C;
    const int o0 = off[b], o1 = off[b + 1];
    const int local = u - o0;
    d.k = (o1 - o0 - bonus_units(C, greedy)) / C;
    if (local < d.k * C) {
        d.i = local / C;
        d.c = local - d.i * C;
    } else {
        d.i = d.k;
        d.c = greedy ? local - d.k * C : 2 * (local - d.k * C);
    }
    d.tr = b * (P.K + 1) + d.i;
    d.e0 = d.c * P.CE;
    d.n = min(P.CE, P.V - d.e0);
    d.drafted = !greedy && d.i < d.k;
    d.pair = !greedy && d.i == d.k && d.c + 1 < C;
    d.has_d = d.drafted || d.pair;
    d.n2 = d.pair ? min(P.CE, P.V - d.e0 - P.CE) : d.n;
    return d;
}

// A unit's two row segments as a data thread loads them: group j of data
// thread dt holds the W elements from (dt + j * kDataThreads) * W.
template <typename E>
struct UnitRows {
    const E* bt;       // target row segment
    const E* bd;       // drafter row segment, or a pair's next target chunk (null: not read)
    int n, nd;         // segment lengths
    bool vt, vd;       // 16-byte loads are legal
};

template <typename E>
__device__ __forceinline__ UnitRows<E> unit_rows(const Params& P, const Unit& d) {
    const E* target = static_cast<const E*>(P.target);
    const E* draft = static_cast<const E*>(P.draft);
    UnitRows<E> w;
    w.bt = target + ((size_t)d.b * (P.K + 1) + d.i) * (size_t)P.V + d.e0;
    w.bd = d.drafted ? draft + ((size_t)d.b * P.K + d.i) * (size_t)P.V + d.e0
         : d.pair    ? w.bt + P.CE
                     : nullptr;
    w.n = d.n;
    w.nd = d.n2;
    w.vt = aligned16(w.bt);
    w.vd = d.has_d && aligned16(w.bd);
    return w;
}

// Data thread dt: issue group j's loads of a unit (no wait).
template <typename E, bool kVec>
__device__ __forceinline__ void load_pair(const UnitRows<E>& w, int dt, int j, uint4& t, uint4& q) {
    constexpr int W = Elem<E>::W;
    const int e = (dt + j * kDataThreads) * W;
    t = e < w.n ? load_group<E, kVec>(w.bt, e, w.n, w.vt) : neg_group<E>();
    q = (w.bd != nullptr && e < w.nd) ? load_group<E, kVec>(w.bd, e, w.nd, w.vd) : neg_group<E>();
}

// Data waves: issue the 16-byte loads of a unit into registers (no wait).
template <typename E, bool kVec, int NG>
__device__ __forceinline__ void issue_loads(const Params& P, const Unit& d, int dt,
                                            uint4 (&gt)[NG], uint4 (&gd)[NG]) {
    const UnitRows<E> w = unit_rows<E>(P, d);
    #pragma unroll
    for (int j = 0; j < NG; ++j) load_pair<E, kVec>(w, dt, j, gt[j], gd[j]);
}

// Control wave: collect the data waves' statistics of the unit of round r,
// merge them and publish them (no wait): sampled, the unit's record
// (epoch-tagged words); greedy, the chunk's argmax key to its team's key.
template <typename E, bool kGreedy>
__device__ __forceinline__ void control_unit(const Params& P, Shared& sh, const Unit& cur, int r) {
    const int lane = threadIdx.x & 63;
    const int C = P.C;
    const int slot = r % kMbox;
    const unsigned ep = P.epoch;
    // Sampled, a drafted position: the drafted token's logits when this
    // chunk holds it (the loads go out before the wait below).
    bool has_x = false;
    float zt = 0.0f, zd = 0.0f;
    if (!kGreedy && cur.drafted) {
        const int x = P.tokens[(size_t)cur.b * P.K + cur.i];
        has_x = x >= cur.e0 && x < cur.e0 + cur.n;
        if (has_x) {
            const E* target = static_cast<const E*>(P.target);
            const E* draft = static_cast<const E*>(P.draft);
            zt = Elem<E>::one(target + ((size_t)cur.b * (P.K + 1) + cur.i) * (size_t)P.V + x);
            zd = Elem<E>::one(draft + ((size_t)cur.b * P.K + cur.i) * (size_t)P.V + x);
        }
    }
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
        wave_argmax(bv, bi);
        if (lane == 0 && bi != INT_MAX) max64(team_key(P, cur.tr), arg_key(bv, bi));
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
        // Rescale each wave's sum from its own maximum to the chunk maximum
        // (both scaled by c).
        if (a > 0.0) a *= (double)fast_exp2(mt - Mt);
        if (d > 0.0) d *= (double)fast_exp2(md - Md);
        const double St = wave_sum(a), Sd = wave_sum(d);
        if (lane == 0 && cur.pair) {
            // Two chunks of the bonus row: chunk c's statistics, then chunk
            // c + 1's from the second registers (no drafter row).
            st64(rec + R_MT, tagged(Mt, ep));
            st64(rec + R_MD, tagged(-INFINITY, ep));
            st64(rec + R_ST, tagged((float)St, ep));
            st64(rec + R_SD, tagged(0.0f, ep));
            st64(rec + kRecWords + R_MT, tagged(Md, ep));
            st64(rec + kRecWords + R_MD, tagged(-INFINITY, ep));
            st64(rec + kRecWords + R_ST, tagged((float)Sd, ep));
            st64(rec + kRecWords + R_SD, tagged(0.0f, ep));
        } else if (lane == 0) {
            st64(rec + R_MT, tagged(Mt, ep));
            st64(rec + R_MD, tagged(Md, ep));
            st64(rec + R_ST, tagged((float)St, ep));
            st64(rec + R_SD, tagged((float)Sd, ep));
            if (has_x) {
                st64(rec + R_ZT, tagged(zt, ep));
                st64(rec + R_ZD, tagged(zd, ep));
            }
        }
    }
}

// -------------------------------------------------------------- planning --

// The request of unit u (off[b] <= u < off[b + 1]; every request has at
// least one unit, so the offsets increase strictly) by a 64-ary search over
// the offsets in LDS. Control wave; uniform result.
__device__ int request_of(const Params& P, const int* off, int u) {
    const int lane = threadIdx.x & 63;
    int lo = 0, n = P.B;                 // off[lo] <= u < off[lo + n]
    while (n > 1) {
        const int step = (n + 63) >> 6;
        const bool le = lane * step < n && off[lo + lane * step] <= u;
        const unsigned long long m = __ballot(le);            // lane 0 always holds
        const int last = 63 - __clzll((long long)m);
        lo += last * step;
        n = min(step, n - last * step);
    }
    return lo;
}

// Control wave: write the plan of data round q: unit u of the sequence, or
// the end of the loop (u >= U).
__device__ __forceinline__ void plan_round(const Params& P, Shared& sh, const int* off, int q,
                                           int u, int U) {
    const int slot = q % kPlanSlots;
    const bool unit = u < U;
    const int b = unit ? request_of(P, off, u) : 0;
    if ((threadIdx.x & 63) == 0) {
        sh.pl_u[slot] = u;
        sh.pl_b[slot] = b;
        sh.pl_kind[slot] = unit ? PL_UNIT : PL_END;
        order();
        lds_put(&sh.pl_tag[slot], q);
    }
}

// Greedy: a unit that was counted on its request's counter (old = the
// counter's value before). Its workgroup completes the request once old
// shows that this unit was the request's last.
struct Pending {
    int b, k, n;        // request, budget, units of the request
    unsigned old;
    bool valid;
};

// The control wave's loop. Units are handed out dynamically: the first
// kPlanLead rounds of workgroup w take units w, w + G, w + 2G, ...; later
// rounds take the values of a device-scope counter (from kPlanLead * G on),
// one fetch in flight at a time, so a workgroup that runs faster takes more
// units and the units of one team are taken, and finish, close together in
// time. Every round:
//  P. plan round r + kPlanLead from the fetched value, and fetch the next;
//  1. the data waves' results of round r: the unit's statistics are merged
//     and published (greedy: posted to the team's key);
//  2. greedy: the unit counted last round: if it was its request's last,
//     complete the request;
//  3. greedy: count this unit on its request's counter (after its key is
//     posted); the returned count is read next round.
// Sampled, the records are all the pass leaves: the draw pass decides the
// drafted positions. No step waits on another workgroup: a greedy request
// is decided by whichever workgroup counts its last unit, so the loop never
// depends on which workgroups are resident. Nothing the data waves do waits
// on a decision.
template <typename E, bool kGreedy, bool kVec>
__device__ __forceinline__ void control_loop(const Params& P, Shared& sh, const int* off) {
    const int U = off[P.B];
    const int G = (int)gridDim.x;
    const int base = kPlanLead * G;
    int planned = 0, end_round = INT_MAX;
    for (int q = 0; q < kPlanLead && end_round == INT_MAX; ++q) {
        const int u = (int)blockIdx.x + q * G;
        plan_round(P, sh, off, planned++, u, U);
        if (u >= U) end_round = q;
    }
    // Device-scope counters are fetched by lane 0 only; its value is made
    // uniform where it is used (the wait for the atomic falls there).
    const int lane = threadIdx.x & 63;
    unsigned fetched = 0;
    if (lane == 0) {
        // Clear the counter the previous launch used, for the next one.
        if (blockIdx.x == 0) st32(P.sched + ((P.epoch & 1u) ? SC_NEXT0 : SC_NEXT1), 0u);
        if (end_round == INT_MAX) fetched = add32(sched_next(P), 1u);
    }
    Pending pend;
    pend.valid = false;
    auto settle = [&]() __attribute__((always_inline)) {
        if (pend.valid &&
            (unsigned)__builtin_amdgcn_readfirstlane((int)pend.old) == (unsigned)(pend.n - 1)) {
            request_complete(P, pend.b, pend.k);
        }
        pend.valid = false;
    };
    for (int r = 0; r < end_round; ++r) {
        // P.
        if (end_round == INT_MAX && r + kPlanLead == planned) {
            const long long u64 =
                (long long)base + (unsigned)__builtin_amdgcn_readfirstlane((int)fetched);
            const int u = u64 < U ? (int)u64 : U;
            plan_round(P, sh, off, planned, u, U);
            if (u >= U) {
                end_round = planned;
            } else if (lane == 0) {
                fetched = add32(sched_next(P), 1u);
            }
            ++planned;
        }
        // 1.
        const int slot = r % kPlanSlots;
        const Unit cur = unit_from(P, off, sh.pl_u[slot], sh.pl_b[slot], kGreedy);
        control_unit<E, kGreedy>(P, sh, cur, r);
        // 2.
        settle();
        // 3.
        if (kGreedy) {
            pend.b = cur.b;
            pend.k = cur.k;
            pend.n = request_units(cur.k, P.C, true);
            drain();                                   // the key's maximum is performed first
            pend.old = 0;
            if (lane == 0) pend.old = add32(&P.req_count[cur.b * kReqStride], 1u);
            pend.valid = true;
        }
    }
    settle();
}

// The data waves' loop: each round reads its plan, reduces the unit in
// registers, issues the loads of the next planned round, and posts its
// results to the control wave.
template <typename E, bool kGreedy, bool kVec>
__device__ __forceinline__ void data_loop(const Params& P, Shared& sh, const int* off) {
    constexpr int W = Elem<E>::W;
    const int lane = threadIdx.x & 63;
    const int dw = (threadIdx.x >> 6) - 1;         // data wave index
    const int dt = threadIdx.x - 64;               // data thread index
    const float cs = P.c32;

    // The plan of round q (the control wave wrote it long before).
    auto read_plan = [&](int q, Unit& u, int& kind) __attribute__((always_inline)) {
        const int slot = q % kPlanSlots;
        lds_wait(P, sh, &sh.pl_tag[slot], q);
        kind = sh.pl_kind[slot];
        u = unit_from(P, off, kind == PL_END ? -1 : sh.pl_u[slot], sh.pl_b[slot], kGreedy);
    };

    constexpr int NG = groups_of<kGreedy>();
    uint4 gt[NG], gd[NG];
    Unit cur;
    int kind;
    read_plan(0, cur, kind);
    if (kind == PL_END) return;
    issue_loads<E, kVec, NG>(P, cur, dt, gt, gd);
    for (int r = 0;; ++r) {
        const int slot = r % kMbox;
        Unit nxt;
        int nkind;
        double post_a = 0.0, post_b = 0.0;
        float post_mt = -INFINITY, post_md = -INFINITY;
        int post_idx = INT_MAX;
        if (kGreedy) {
            float bv = -INFINITY;
            int bi = INT_MAX;
            // Group by group; a consumed group's registers take the next
            // unit's group at once.
            read_plan(r + 1, nxt, nkind);
            const bool more = nkind != PL_END;
            UnitRows<E> nw;
            if (more) nw = unit_rows<E>(P, nxt);
            #pragma unroll
            for (int j = 0; j < NG; ++j) {
                #pragma unroll
                for (int kk = 0; kk < W; ++kk) {
                    const float v = Elem<E>::at(gt[j], kk);
                    if (v > bv) {                  // a lane's elements go up in index order
                        bv = v;
                        bi = cur.e0 + (dt + j * kDataThreads) * W + kk;
                    }
                }
                if (more) load_pair<E, kVec>(nw, dt, j, gt[j], gd[j]);
            }
            wave_argmax_xbar(bv, bi);
            post_mt = bv;
            post_idx = bi;
        } else {
            float mt = -INFINITY, md = -INFINITY;
            #pragma unroll
            for (int j = 0; j < NG; ++j) {
                #pragma unroll
                for (int kk = 0; kk < W; ++kk) {
                    mt = fmaxf(mt, Elem<E>::at(gt[j], kk));
                    md = fmaxf(md, Elem<E>::at(gd[j], kk));
                }
            }
            // Opaque raw registers: the exp pass converts them again rather
            // than keeping every converted float alive across the reduction.
            #pragma unroll
            for (int j = 0; j < NG; ++j) {
                asm volatile("" : "+v"(gt[j].x), "+v"(gt[j].y), "+v"(gt[j].z), "+v"(gt[j].w));
                asm volatile("" : "+v"(gd[j].x), "+v"(gd[j].y), "+v"(gd[j].z), "+v"(gd[j].w));
            }
            mt = wave_max_xbar(mt);
            md = wave_max_xbar(md);
            // Exp pass, group by group; as soon as a group is consumed its
            // registers take the next unit's group (loads overlap the rest
            // of the pass).
            read_plan(r + 1, nxt, nkind);
            const bool more = nkind != PL_END;
            UnitRows<E> nw;
            if (more) nw = unit_rows<E>(P, nxt);
            const bool do_t = mt != -INFINITY, do_d = cur.has_d && md != -INFINITY;
            // Maxima in scaled units (s = m c, rounded once); each term is
            // 2^(z c - s), one fused multiply-add and an exp2.
            const float smt = mt * cs, smd = md * cs;
            float lt = 0.0f, ld = 0.0f;
            #pragma unroll
            for (int j = 0; j < NG; ++j) {
                float e[W], f[W];
                #pragma unroll
                for (int kk = 0; kk < W; ++kk) {
                    e[kk] = do_t ? fast_exp2(__builtin_fmaf(Elem<E>::at(gt[j], kk), cs, -smt)) : 0.0f;
                    f[kk] = do_d ? fast_exp2(__builtin_fmaf(Elem<E>::at(gd[j], kk), cs, -smd)) : 0.0f;
                }
                if (more) load_pair<E, kVec>(nw, dt, j, gt[j], gd[j]);
                #pragma unroll
                for (int h = W / 2; h > 0; h >>= 1) {
                    #pragma unroll
                    for (int kk = 0; kk < h; ++kk) {
                        e[kk] += e[kk + h];
                        f[kk] += f[kk + h];
                    }
                }
                lt += e[0];
                ld += f[0];
            }
            post_a = wave_sum_xbar((double)lt);
            post_b = wave_sum_xbar((double)ld);
            post_mt = smt;
            post_md = smd;
        }
        if (lane == 0) {
            if (r >= kMbox) lds_wait(P, sh, &sh.st_done[slot], r - kMbox + 1);
            sh.st_mt[slot][dw] = post_mt;
            sh.st_md[slot][dw] = post_md;
            sh.st_st[slot][dw] = post_a;
            sh.st_sd[slot][dw] = post_b;
            sh.st_idx[slot][dw] = post_idx;
            order();
            lds_put(&sh.st_tag[slot][dw], r + 1);
        }
        if (nkind == PL_END) break;
        cur = nxt;
        kind = nkind;
    }
}

template <typename E, bool kGreedy, bool kVec>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(4)))
void verify_kernel(Params P) {
    extern __shared__ __align__(16) unsigned char dyn_smem[];
    __shared__ Shared sh;
    int* off = reinterpret_cast<int*>(dyn_smem);   // request unit offsets [B + 1]

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
            local += request_units(k, C, kGreedy);
        }
        if (bad && blockIdx.x == 0) atomicOr(P.status, SV_FLAG_BAD_BUDGET);
        int incl = local;
        #pragma unroll
        for (int o = 1; o < 64; o <<= 1) {
            const int v = __shfl_up(incl, o, 64);
            if (lane >= o) incl += v;
        }
        if (lane == 63) sh.red_i[wave] = incl;
        if (tid < kMbox * kDataWaves) (&sh.st_tag[0][0])[tid] = 0;
        if (tid < kMbox) sh.st_done[tid] = 0;
        if (tid < kPlanSlots) sh.pl_tag[tid] = -1;
        if (tid == 0) sh.abort_wait = 0;
        __syncthreads();
        int run = incl - local;
        for (int w = 0; w < wave; ++w) run += sh.red_i[w];
        for (int b = b0; b < b1; ++b) {
            off[b] = run;
            int k = P.budgets[b];
            k = k < 0 ? 0 : (k > K ? K : k);
            run += request_units(k, C, kGreedy);
        }
        if (tid == kThreads - 1) off[B] = run;
        __syncthreads();
    }

    // Wave specialisation (the branch is uniform per wave); no barrier
    // after it.
    if (__builtin_amdgcn_readfirstlane(wave) == 0) {
        control_loop<E, kGreedy, kVec>(P, sh, off);
    } else {
        data_loop<E, kGreedy, kVec>(P, sh, off);
    }
}

// ------------------------------------------------------------- draw pass --

// Wave 0: the chunk of team tr's target row (records in pl, normalisers ts)
// where the running p mass, chunk by chunk, first exceeds u times the row's
// total; thr = the part of that threshold inside the chunk. chunk -1: no
// mass.
__device__ void p_chunk(const Params& P, const TeamPoll& pl, const TeamStats& ts, double u,
                        int& chunk, double& thr) {
    const int lane = threadIdx.x & 63;
    const int C = P.C;
    unsigned long long* rec = team_rec(P, pl.tr);
    chunk = -1;
    thr = 0.0;
    if (!(ts.st > 0.0)) return;
    const double inv = 1.0 / ts.st;
    // Chunk cc's words: lane cc holds them for cc < 64.
    auto pmass = [&](int cc) -> double {
        const float s1 = tag_val(cc == lane ? pl.w[R_ST] : ld64(rec + cc * kRecWords + R_ST));
        const float m1 = tag_val(cc == lane ? pl.w[R_MT] : ld64(rec + cc * kRecWords + R_MT));
        return s1 > 0.0f ? (double)s1 * exp2((double)m1 - (double)ts.mt) * inv : 0.0;
    };
    double total = 0.0;
    for (int cc = lane; cc < C; cc += 64) total += pmass(cc);
    total = wave_sum(total);
    double base = 0.0;
    chunk_crossing(C, u * total, pmass, chunk, base);
    thr = u * total - base;
}

// Sampled mode, second pass: one workgroup per request, launched after the
// streaming pass on the same stream, so every record is final. Wave w
// decides drafted positions w, w + 8, ...: it merges the position's target
// and drafter records into their normalisers, reads the drafted token's two
// logits from the record of the chunk holding it and takes the accept test.
// The deciding position j is the first rejected one (k if all k were
// accepted); wave 0 takes its normalisers and the sampling uniform u. The draw is an inverse
// CDF in vocabulary order over blocks of 64 groups (512 bf16 or 256 fp32
// elements, one 16-byte load per lane): the data waves stream the blocks of
// a range, wave d taking every (kDrawDataWaves)-th block with kDrawSlots
// blocks in flight, and leave each block's mass in LDS; wave 0 finds the
// block where the running mass first exceeds the threshold, and one data
// wave scans that block's elements again (cache-resident).
//  * First rejection (j < k): the residual max(0, p_j - q_j) over the whole
//    row pair, threshold u R. The first blocks' loads go out as soon as the
//    decisions name j.
//  * Bonus position (j == k), or a residual without mass (rounding only):
//    p_j. Its chunk masses follow from the records; the blocks of the chunk
//    holding u times the total are streamed.
// Eight waves per workgroup and two workgroups per CU, so one request's
// start-up and final scan overlap another's streaming.
constexpr int kDrawWaves = 8;                  // wave 0: control; waves 1-7: data
constexpr int kDrawThreads = kDrawWaves * 64;
constexpr int kDrawDataWaves = kDrawWaves - 1;
constexpr int kDrawSlots = 5;                  // blocks in flight per data wave
constexpr int kDrawNone = 0, kDrawResidual = 1, kDrawP = 2;

// Draw pass state, written between barriers: the decisions by the waves
// that take them, the rest by wave 0.
struct DrawShared {
    int mode;          // kDrawNone, kDrawResidual or kDrawP
    int x0, x1;        // block range streamed
    int star;          // block holding the threshold, from x0 (-1: none)
    int done;          // star found
    int last;          // this workgroup finished a request's masses last
    int y;             // drawn token
    double u;          // sampling uniform of position j
    double thr;        // threshold, as mass from block x0's start (then from block star's)
    float mt, md, ist, isd;
    // The decisions: drafted position t's accept bit and its rows' normalisers.
    int acc[SV_MAX_K];
    float tmt[SV_MAX_K], tmd[SV_MAX_K];
    double tst[SV_MAX_K], tsd[SV_MAX_K];
};

constexpr int kDecPer = (SV_MAX_K + kDrawWaves - 1) / kDrawWaves;   // positions per wave

template <typename E, bool kVec>
__global__ __launch_bounds__(kDrawThreads) __attribute__((amdgpu_waves_per_eu(4)))
void draw_kernel(Params P) {
    extern __shared__ __align__(16) unsigned char dyn_smem[];
    __shared__ DrawShared dsh;
    double* blk = reinterpret_cast<double*>(dyn_smem);   // block masses of the range [x0, x1)
    constexpr int W = Elem<E>::W;
    constexpr int BE = 64 * W;                           // elements per block
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    // Requests in reverse order: the streaming pass read the last requests'
    // rows last, so they are the likeliest to still be cached. With a split
    // (small batches), workgroup sl of a request takes the sl-th of dsplit
    // slices of its blocks; the slices of one request are B workgroups apart.
    const int S = P.dsplit;
    const int b = P.B - 1 - (int)(blockIdx.x % (unsigned)P.B);
    const int sl = (int)(blockIdx.x / (unsigned)P.B);
    const int K = P.K, V = P.V;
    const int NB = (V + BE - 1) / BE;                    // blocks per row
    const unsigned ep = P.epoch;
    // The decisions. Wave w takes drafted positions w, w + 8, ... below the
    // budget: one round of loads brings the budget, each position's drafted
    // token and the records of its target and drafter rows (their maxima,
    // sums and the token's logits, which the chunk holding the token
    // recorded); then p(x), q(x) and the accept test, as the pages' rule has
    // them, with the Philox uniform of (b, t).
    const int C = P.C;
    int k = P.budgets[b];
    TeamPoll dpl[kDecPer];
    unsigned long long dzt[kDecPer], dzd[kDecPer];
    int dx[kDecPer];
    #pragma unroll
    for (int u = 0; u < kDecPer; ++u) {
        const int t = wave + u * kDrawWaves;
        dzt[u] = dzd[u] = 0ull;
        dx[u] = -1;
        if (t < K) {
            poll_issue(P, b * (K + 1) + t, dpl[u]);
            unsigned long long* rec = team_rec(P, b * (K + 1) + t);
            if (lane < C) {
                dzt[u] = ld64(rec + lane * kRecWords + R_ZT);
                dzd[u] = ld64(rec + lane * kRecWords + R_ZD);
            }
            dx[u] = P.tokens[(size_t)b * K + t];
        }
    }
    k = k < 0 ? 0 : (k > K ? K : k);
    #pragma unroll
    for (int u = 0; u < kDecPer; ++u) {
        const int t = wave + u * kDrawWaves;
        if (t < k) {
            const int tr = b * (K + 1) + t;
            if (!poll_complete(P, dpl[u]) && lane == 0) atomicOr(P.status, SV_FLAG_SYNC_TIMEOUT);
            const TeamStats ts = team_stats(P, dpl[u]);
            const int x = dx[u];
            const bool valid = x >= 0 && x < V;
            double px = 0.0, qx = 0.0;
            if (valid) {
                const int cx = x / P.CE;
                unsigned long long wt, wd;
                if (cx < 64) {
                    wt = (unsigned long long)__shfl((long long)dzt[u], cx, 64);
                    wd = (unsigned long long)__shfl((long long)dzd[u], cx, 64);
                } else {
                    unsigned long long* rec = team_rec(P, tr);
                    wt = ld64(rec + cx * kRecWords + R_ZT);
                    wd = ld64(rec + cx * kRecWords + R_ZD);
                }
                if ((!tag_ok(wt, ep) || !tag_ok(wd, ep)) && lane == 0) {
                    atomicOr(P.status, SV_FLAG_SYNC_TIMEOUT);
                }
                // z c exactly (a product of two fp32 values fits fp64), minus
                // the scaled maximum the row's sum was taken under.
                px = exp2((double)tag_val(wt) * (double)P.c32 - (double)ts.mt) / ts.st;
                qx = exp2((double)tag_val(wd) * (double)P.c32 - (double)ts.md) / ts.sd;
            }
            const uint4 rw = philox4x32_10(P.bbase + (uint32_t)b, (uint32_t)t, 0u, 0u, P.key0, P.key1);
            const bool accept = word_to_uniform(rw.x) * qx < px;
            if (lane == 0) {
                if (!valid) atomicOr(P.status, SV_FLAG_BAD_TOKEN);
                if (sl == 0) {
                    if (P.out_p) P.out_p[(size_t)b * K + t] = (float)px;
                    if (P.out_q) P.out_q[(size_t)b * K + t] = (float)qx;
                }
                dsh.acc[t] = accept ? 1 : 0;
                dsh.tmt[t] = ts.mt;
                dsh.tmd[t] = ts.md;
                dsh.tst[t] = ts.st;
                dsh.tsd[t] = ts.sd;
            }
        }
    }
    if (tid == 0) {
        dsh.done = 0;
        dsh.last = 0;
        dsh.y = 0;
    }
    __syncthreads();
    // The first rejected drafted position (k if none): the residual's, or
    // the bonus position.
    int j = k;
    for (int t = 0; t < k; ++t) {
        if (dsh.acc[t] == 0) {
            j = t;
            break;
        }
    }
    TeamPoll pl;                                         // wave 0, bonus: team k's records
    if (wave == 0 && j == k) poll_issue(P, b * (K + 1) + j, pl);
    const E* rt = static_cast<const E*>(P.target) + ((size_t)b * (K + 1) + j) * (size_t)V;
    const E* rd = j < k ? static_cast<const E*>(P.draft) + ((size_t)b * K + j) * (size_t)V : nullptr;
    const bool vt = aligned16(rt), vd = rd != nullptr && aligned16(rd);
    const int dw = wave - 1;
    const int stride = kDrawSlots * kDrawDataWaves;      // blocks between a slot's loads

    // Block x's group of this lane: elements (x * 64 + lane) * W onwards;
    // past V they read as -inf (zero mass).
    uint4 gt[kDrawSlots], gd[kDrawSlots];
    auto issue = [&](int x, bool res, uint4& t, uint4& q) __attribute__((always_inline)) {
        const int e = (x * 64 + lane) * W;
        t = load_group<E, kVec>(rt, e, V, vt);
        if (res) q = load_group<E, kVec>(rd, e, V, vd);
    };
    auto preload = [&](int x0, int x1, bool res) __attribute__((always_inline)) {
        #pragma unroll
        for (int s = 0; s < kDrawSlots; ++s) {
            const int x = x0 + dw + s * kDrawDataWaves;
            if (x < x1) issue(x, res, gt[s], gd[s]);
        }
    };
    // This workgroup's slice of a block range in the first round.
    auto slice = [&](int x0, int x1, int& a0, int& a1) __attribute__((always_inline)) {
        const int n = x1 - x0;
        a0 = x0 + (int)(((long long)sl * n) / S);
        a1 = x0 + (int)(((long long)(sl + 1) * n) / S);
    };
    bool pre = false;
    if (j < k && wave > 0) {
        int a0, a1;
        slice(0, NB, a0, a1);
        preload(a0, a1, true);
        pre = true;
    }
    if (wave == 0) {
        // The drawn row's normalisers: the residual's from the decisions,
        // the bonus row's from its records.
        TeamStats ts;
        if (j < k) {
            ts.mt = dsh.tmt[j];
            ts.md = dsh.tmd[j];
            ts.st = dsh.tst[j];
            ts.sd = dsh.tsd[j];
        } else {
            if (!poll_complete(P, pl) && lane == 0) atomicOr(P.status, SV_FLAG_SYNC_TIMEOUT);
            ts = team_stats(P, pl);
        }
        const uint4 rw = philox4x32_10(P.bbase + (uint32_t)b, (uint32_t)j, 0u, 0u, P.key0, P.key1);
        const double u = word_to_uniform(rw.y);
        int x0 = 0, x1 = NB, mode = j < k ? kDrawResidual : kDrawP;
        double thr = 0.0;
        if (mode == kDrawP) {
            int chunk = -1;
            p_chunk(P, pl, ts, u, chunk, thr);
            if (chunk < 0) {
                mode = kDrawNone;
            } else {
                x0 = chunk * kBlocks;
                x1 = min(x0 + kBlocks, NB);
            }
        }
        if (lane == 0) {
            dsh.mode = mode;
            dsh.x0 = x0;
            dsh.x1 = x1;
            dsh.u = u;
            dsh.thr = thr;
            dsh.mt = ts.mt;
            dsh.md = ts.md;
            dsh.ist = (float)(1.0 / ts.st);
            dsh.isd = (float)(1.0 / ts.sd);
        }
    }
    __syncthreads();
    const float mt = dsh.mt, md = dsh.md, ist = dsh.ist, isd = dsh.isd;
    const float c = P.c32;
    // p = 2^(z c - s_t) / S_t and q likewise, with the scaled maxima the
    // sums were taken under.
    auto mass = [&](const uint4& t, const uint4& q, int kk, bool res) -> float {
        const float pv = fast_exp2(__builtin_fmaf(Elem<E>::at(t, kk), c, -mt)) * ist;
        if (!res) return pv;
        return fmaxf(0.0f, pv - fast_exp2(__builtin_fmaf(Elem<E>::at(q, kk), c, -md)) * isd);
    };
    // At most two rounds: the residual, then p_j if the residual had no mass.
    // Only the first is split over workgroups; the fallback runs in the
    // workgroup that finished the first round last.
    for (int round = 0; round < 2; ++round) {
        const int mode = dsh.mode;
        if (mode == kDrawNone) break;
        const bool res = mode == kDrawResidual;
        const int x0 = dsh.x0, x1 = dsh.x1;
        const bool split = round == 0 && S > 1;
        int a0 = x0, a1 = x1;
        if (split) slice(x0, x1, a0, a1);
        double* gm = P.dmass + (size_t)b * (size_t)(P.C * kBlocks);
        if (wave > 0) {
            if (!(pre && round == 0)) preload(a0, a1, res);
            for (int xr = a0 + dw; xr < a1; xr += stride) {
                #pragma unroll
                for (int s = 0; s < kDrawSlots; ++s) {
                    const int x = xr + s * kDrawDataWaves;
                    if (x < a1) {
                        float sg = 0.0f;
                        #pragma unroll
                        for (int kk = 0; kk < W; ++kk) sg += mass(gt[s], gd[s], kk, res);
                        const double ws = wave_sum_xbar((double)sg);
                        if (lane == 0) {
                            blk[x - x0] = ws;
                            if (split) {
                                st64(reinterpret_cast<unsigned long long*>(gm + (x - x0)),
                                     (unsigned long long)__double_as_longlong(ws));
                            }
                        }
                        if (x + stride < a1) issue(x + stride, res, gt[s], gd[s]);
                    }
                }
            }
            // The published masses are complete before the count below.
            if (split) drain();
        }
        if (split) {
            __syncthreads();
            if (tid == 0) {
                const unsigned old = add32(&P.dcnt[(size_t)b * kReqStride], 1u);
                const int last = old == (unsigned)(S - 1);
                // Every slice of the request has been counted: reset for the
                // next call.
                if (last) st32(&P.dcnt[(size_t)b * kReqStride], 0u);
                dsh.last = last;
            }
            __syncthreads();
            if (!dsh.last) return;                          // another workgroup finishes
            for (int x = tid; x < x1 - x0; x += kDrawThreads) {
                blk[x] = __longlong_as_double(
                    (long long)ld64(reinterpret_cast<unsigned long long*>(gm + x)));
            }
        }
        __syncthreads();
        if (wave == 0) {
            const int nb = x1 - x0;
            double thr = dsh.thr;
            bool any = true;
            if (res) {
                double total = 0.0;
                for (int x = lane; x < nb; x += 64) total += blk[x];
                total = wave_sum(total);
                thr = dsh.u * total;
                any = total > 0.0;
            }
            int star = -1;
            double base = 0.0;
            if (any) chunk_crossing(nb, thr, [&](int x) -> double { return blk[x]; }, star, base);
            int nmode = mode, nx0 = x0, nx1 = x1;
            double nthr = thr - base;
            if (star < 0) {
                nmode = kDrawNone;
                if (res) {
                    // No residual mass (rounding only): from p_j, whose
                    // records are read again.
                    TeamPoll pr;
                    poll_issue(P, b * (K + 1) + j, pr);
                    const TeamStats tr = team_stats(P, pr);
                    int chunk = -1;
                    p_chunk(P, pr, tr, dsh.u, chunk, nthr);
                    if (chunk >= 0) {
                        nmode = kDrawP;
                        nx0 = chunk * kBlocks;
                        nx1 = min(nx0 + kBlocks, NB);
                    }
                }
            }
            if (lane == 0) {
                dsh.star = star;
                dsh.done = star >= 0;
                dsh.mode = nmode;
                dsh.x0 = nx0;
                dsh.x1 = nx1;
                dsh.thr = nthr;
            }
        }
        __syncthreads();
        if (dsh.done) break;
    }
    if (dsh.done) {
        if (wave == 1) {
            // The block's elements again, in order: the first whose running
            // mass exceeds the threshold; zero-mass elements are never drawn.
            const bool res = dsh.mode == kDrawResidual;
            const int x = dsh.x0 + dsh.star;
            uint4 t4, q4;
            issue(x, res, t4, q4);
            const int e = (x * 64 + lane) * W;
            float r[W];
            double pref[W];
            double run = 0.0;
            #pragma unroll
            for (int kk = 0; kk < W; ++kk) {
                r[kk] = mass(t4, q4, kk, res);
                run += (double)r[kk];
                pref[kk] = run;
            }
            const double incl = wave_incl_scan(run, lane);
            const double up = __shfl_up(incl, 1, 64);
            const double excl = lane ? up : 0.0;
            const double tt = dsh.thr;
            int cand = INT_MAX, last = -1;
            #pragma unroll
            for (int kk = 0; kk < W; ++kk) {
                if (r[kk] > 0.0f) {
                    last = e + kk;
                    if (cand == INT_MAX && excl + pref[kk] > tt) cand = e + kk;
                }
            }
            #pragma unroll
            for (int o = 32; o > 0; o >>= 1) {
                cand = min(cand, __shfl_xor(cand, o, 64));
                last = max(last, __shfl_xor(last, o, 64));
            }
            if (lane == 0) dsh.y = cand != INT_MAX ? cand : (last >= 0 ? last : 0);
        }
        __syncthreads();
    }
    // With no draw (no mass anywhere), the first slice writes the outputs.
    if (tid == 0 && (dsh.done || dsh.last || sl == 0)) request_outputs<false>(P, b, k, j, dsh.y);
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

// Elements per chunk, and chunks per row: sampled (the records and the draw
// pass's blocks are laid out by these), or greedy.
int chunk_elems(int dtype, bool greedy = false) {
    return kDataThreads * (greedy ? groups_of<true>() : groups_of<false>()) * elems_per_group(dtype);
}

int chunks_for(int vocab, int dtype, bool greedy = false) {
    const int ce = chunk_elems(dtype, greedy);
    return (vocab + ce - 1) / ce;
}

size_t dyn_smem_bytes(int B) { return (size_t)(B + 1) * sizeof(int); }

// The draw pass keeps one mass per block of a row (at most C chunks of
// kBlocks blocks).
size_t draw_smem_bytes(int C) { return (size_t)C * kBlocks * sizeof(double); }

// Byte offsets of the kernels' device workspace, for launches of up to
// max_batch requests with up to max_k drafted positions and C chunks per row.
// The draw pass splits a request over several workgroups only for batches of
// at most split_reqs requests. The counters must read zero when a call
// starts: the greedy team keys (words TW_KEY, TW_KEY + 1 of each team
// record) and the words in [req, req_end) and [dcnt, dcnt_end), which every
// kernel that raises one leaves at zero when it completes, and the scheduling word of
// the call's epoch parity at status + 64, which the launch before it clears.
// The status word at `status` accumulates device-side flags.
struct WsLayout {
    size_t rec, team, req, req_end, dmass, dcnt, dcnt_end, status, total;
    size_t teams;
    int split_reqs;
};

WsLayout ws_layout(int max_batch, int max_k, int C, int split_reqs) {
    auto round256 = [](size_t x) { return (x + 255) / 256 * 256; };
    const size_t teams = (size_t)max_batch * (max_k + 1);
    WsLayout L;
    size_t o = 0;
    L.rec = o;
    o += round256(teams * C * kRecWords * 8);
    L.team = o;
    o += round256(teams * kTeamWords * 4);
    L.req = o;
    o += round256((size_t)max_batch * kReqStride * 4);
    L.req_end = o;
    L.dmass = o;
    o += round256((size_t)split_reqs * C * kBlocks * 8);
    L.dcnt = o;
    o += round256((size_t)split_reqs * kReqStride * 4);
    L.dcnt_end = o;
    L.status = o;
    o += 256;
    L.total = o;
    L.teams = teams;
    L.split_reqs = split_reqs;
    return L;
}

// Launch facts of one device: CUs and, per instantiation of the streaming
// pass, the resident workgroups per CU (cached by dynamic LDS size).
struct DeviceInfo {
    int cus;
    size_t occ_smem[8];
    int occ_val[8];
};

int device_info(int device, DeviceInfo& di) {
    std::memset(&di, 0, sizeof(di));
    if (hipDeviceGetAttribute(&di.cus, hipDeviceAttributeMultiprocessorCount, device) !=
            hipSuccess || di.cus < 1) {
        return SV_ERR_HIP;
    }
    return SV_OK;
}

}  // namespace

struct spec_verify_ctx {
    uint32_t magic;
    int device, max_batch, max_k, vocab, dtype;
    int C, CE;
    DeviceInfo info;
    WsLayout lay;
    unsigned char* ws;
    unsigned calls;                // calls made so far (the epochs of its launches)
    // Per-pass timing (off unless enabled): recorded event pairs of later
    // runs, and a pool of events to reuse.
    bool timing;
    struct Timed {
        int pass;                  // 0 streaming pass, 1 draw pass
        hipEvent_t start, end;
    };
    std::vector<Timed> timed;
    std::vector<hipEvent_t> event_pool;
};

namespace {

template <typename E, bool G, bool Vv>
int occupancy_of(DeviceInfo& di, int slot, size_t smem) {
    if (di.occ_smem[slot] == smem && di.occ_val[slot] > 0) return di.occ_val[slot];
    int n = 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, verify_kernel<E, G, Vv>, kThreads, smem) !=
            hipSuccess ||
        n < 1) {
        n = 1;
    }
    di.occ_smem[slot] = smem;
    di.occ_val[slot] = n;
    return n;
}

constexpr size_t kMaxTimed = 1 << 16;   // recorded passes kept before recording stops

hipEvent_t pooled_event(spec_verify_ctx* ctx) {
    if (!ctx->event_pool.empty()) {
        hipEvent_t e = ctx->event_pool.back();
        ctx->event_pool.pop_back();
        return e;
    }
    hipEvent_t e = nullptr;
    return hipEventCreate(&e) == hipSuccess ? e : nullptr;
}

// Start of a pass: when timing, an event pair is taken and its start
// recorded; returns the record's index, or -1. ctx may be null (no timing).
int timed_begin(spec_verify_ctx* ctx, int pass, hipStream_t stream) {
    if (!ctx || !ctx->timing || ctx->timed.size() >= kMaxTimed) return -1;
    spec_verify_ctx::Timed t;
    t.pass = pass;
    t.start = pooled_event(ctx);
    t.end = pooled_event(ctx);
    if (!t.start || !t.end || hipEventRecord(t.start, stream) != hipSuccess) {
        if (t.start) ctx->event_pool.push_back(t.start);
        if (t.end) ctx->event_pool.push_back(t.end);
        return -1;
    }
    ctx->timed.push_back(t);
    return (int)ctx->timed.size() - 1;
}

void timed_end(spec_verify_ctx* ctx, int idx, hipStream_t stream) {
    if (ctx && idx >= 0) (void)hipEventRecord(ctx->timed[(size_t)idx].end, stream);
}

// Launch shape of the streaming pass: every workgroup resident (grid = CUs x
// occupancy); the schedule needs at least as many workgroups as a team has
// members. Sampled mode then runs the draw pass, one workgroup per request.
template <typename E, bool G, bool Vv>
int launch(DeviceInfo& di, spec_verify_ctx* tctx, int split_reqs, Params& p, hipStream_t stream,
           unsigned& calls) {
    const int slot = (std::is_same<E, uint16_t>::value ? 4 : 0) + (G ? 2 : 0) + (Vv ? 1 : 0);
    const size_t smem = dyn_smem_bytes(p.B);
    const int occ = occupancy_of<E, G, Vv>(di, slot, smem);
    const long long grid = (long long)di.cus * occ;
    if (grid < (long long)p.C) return SV_ERR_ARG;   // a team would not fit
    int t = timed_begin(tctx, 0, stream);
    hipLaunchKernelGGL((verify_kernel<E, G, Vv>), dim3((unsigned)grid), dim3(kThreads), smem, stream,
                       p);
    if (hipGetLastError() != hipSuccess) return SV_ERR_HIP;
    calls = p.epoch;                                // the epoch is spent once the pass is enqueued
    timed_end(tctx, t, stream);
    if (!G) {
        // Two draw workgroups fit a CU. A batch of fewer requests than that
        // splits each request's blocks over several workgroups (at least 16
        // blocks each, at most 64 workgroups per request).
        const int nb = (p.V + 64 * Elem<E>::W - 1) / (64 * Elem<E>::W);
        int S = 1;
        if (p.B <= split_reqs) {
            S = (2 * di.cus) / p.B;
            S = S < 1 ? 1 : (S > 64 ? 64 : S);
            const int smax = nb / 16 < 1 ? 1 : nb / 16;
            S = S > smax ? smax : S;
        }
        p.dsplit = S;
        t = timed_begin(tctx, 1, stream);
        hipLaunchKernelGGL((draw_kernel<E, Vv>), dim3((unsigned)(p.B * S)), dim3(kDrawThreads),
                           draw_smem_bytes(p.C), stream, p);
        if (hipGetLastError() != hipSuccess) return SV_ERR_HIP;
        timed_end(tctx, t, stream);
    }
    return SV_OK;
}

bool aligned_to(const void* p, size_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

// The caller's arguments of one verify call (already checked).
struct RunArgs {
    const void* target;
    const void* draft;
    const int32_t* tokens;
    const int32_t* budgets;
    int B, K;
    float temperature;
    uint64_t seed;
    uint32_t request_base;
    int32_t* out_tokens;
    int32_t* out_nacc;
    float* out_p;
    float* out_q;
};

// Enqueue one verify call on the stream: batches beyond kLaunchBatch requests
// run as consecutive launches (each launch keeps its request table in LDS);
// the workspace ws (laid out by L) is reused, and the Philox counter keeps
// the caller's request index. calls: the epoch counter of this workspace.
int run_batches(DeviceInfo& di, spec_verify_ctx* tctx, int vocab, int dtype, unsigned char* ws,
                const WsLayout& L, unsigned& calls, unsigned* status, const RunArgs& a,
                hipStream_t s) {
    const bool greedy = a.temperature == 0.0f;
    const int K = a.K;
    Params p;
    std::memset(&p, 0, sizeof(p));
    p.rec = reinterpret_cast<unsigned long long*>(ws + L.rec);
    p.team = reinterpret_cast<unsigned*>(ws + L.team);
    p.req_count = reinterpret_cast<unsigned*>(ws + L.req);
    p.sched = reinterpret_cast<unsigned*>(ws + L.status + 64);
    p.status = status;
    p.dmass = reinterpret_cast<double*>(ws + L.dmass);
    p.dcnt = reinterpret_cast<unsigned*>(ws + L.dcnt);
    p.K = K;
    p.V = vocab;
    p.C = chunks_for(vocab, dtype, greedy);
    p.CE = chunk_elems(dtype, greedy);
    p.c64 = greedy ? 0.0 : kLog2e / (double)a.temperature;
    p.c32 = (float)p.c64;
    p.key0 = (uint32_t)(a.seed & 0xFFFFFFFFu);
    p.key1 = (uint32_t)(a.seed >> 32);
    // Vector-only loads when every row starts on a 16-byte boundary.
    const size_t es = dtype == SV_DTYPE_BF16 ? 2 : 4;
    const bool vec = aligned_to(a.target, 16) && (greedy || K == 0 || aligned_to(a.draft, 16)) &&
                     ((size_t)vocab * es) % 16 == 0;
    const size_t V = (size_t)vocab;
    int r = SV_OK;
    for (int b0 = 0; b0 < a.B && r == SV_OK; b0 += kLaunchBatch) {
        Params q = p;
        q.B = a.B - b0 < kLaunchBatch ? a.B - b0 : kLaunchBatch;
        q.bbase = a.request_base + (uint32_t)b0;
        q.target = static_cast<const unsigned char*>(a.target) + (size_t)b0 * (K + 1) * V * es;
        q.draft = greedy ? nullptr
                         : static_cast<const unsigned char*>(a.draft) + (size_t)b0 * K * V * es;
        q.tokens = a.tokens ? a.tokens + (size_t)b0 * K : nullptr;
        q.budgets = a.budgets + b0;
        q.out_tokens = a.out_tokens + (size_t)b0 * (K + 1);
        q.out_nacc = a.out_nacc + b0;
        q.out_p = a.out_p ? a.out_p + (size_t)b0 * K : nullptr;
        q.out_q = a.out_q ? a.out_q + (size_t)b0 * K : nullptr;
        // 1 .. 2^32 - 2, never 0; an even cycle, so consecutive launches
        // alternate in parity, across the wrap too.
        q.epoch = calls % 0xFFFFFFFEu + 1u;
        const int sr = L.split_reqs;
        if (dtype == SV_DTYPE_BF16) {
            if (vec) {
                r = greedy ? launch<uint16_t, true, true>(di, tctx, sr, q, s, calls)
                           : launch<uint16_t, false, true>(di, tctx, sr, q, s, calls);
            } else {
                r = greedy ? launch<uint16_t, true, false>(di, tctx, sr, q, s, calls)
                           : launch<uint16_t, false, false>(di, tctx, sr, q, s, calls);
            }
        } else {
            if (vec) {
                r = greedy ? launch<float, true, true>(di, tctx, sr, q, s, calls)
                           : launch<float, false, true>(di, tctx, sr, q, s, calls);
            } else {
                r = greedy ? launch<float, true, false>(di, tctx, sr, q, s, calls)
                           : launch<float, false, false>(di, tctx, sr, q, s, calls);
            }
        }
    }
    return r;
}

// ------------------------------------------------ allocation-free variant --

// The allocation-free entry point's workspace: one static array per device
// (every GPU the library runs on holds its own copy until the process ends).
// In host code `scratch` names a host-side stand-in, never the device memory:
// its device address is taken once per device with hipGetSymbolAddress and
// only that address is used.
static __device__ __align__(256) unsigned char scratch[SV_NOALLOC_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;

struct NoallocDevice {
    bool ready;
    unsigned char* ptr;            // device address of this device's `scratch`
    DeviceInfo info;
    unsigned calls;                // epochs of calls on this device's scratch
};

std::mutex g_noalloc_mu;
NoallocDevice g_noalloc[kMaxDevices];

// Zero the call-start counters of the scratch (a fill kernel rather than a
// memset, so the call can be captured in a HIP graph): the greedy team keys
// (two words every kTeamWords), the request and draw-split counters,
// the scheduling words, and the caller's status word.
__global__ void clear_words_kernel(unsigned* team, int nteam, unsigned* a, int na, unsigned* b,
                                   int nb, unsigned* sched, uint32_t* status) {
    const int t = blockIdx.x * blockDim.x + threadIdx.x;
    const int stride = gridDim.x * blockDim.x;
    for (int i = t; i < nteam; i += stride) {
        team[(size_t)i * kTeamWords + TW_KEY] = 0u;
        team[(size_t)i * kTeamWords + TW_KEY + 1] = 0u;
    }
    for (int i = t; i < na; i += stride) a[i] = 0u;
    for (int i = t; i < nb; i += stride) b[i] = 0u;
    if (t == 0) {
        sched[SC_NEXT0] = 0u;
        sched[SC_NEXT1] = 0u;
        if (status) *status = 0u;
    }
}

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
        case SV_ERR_TOO_BIG:
            return "the call needs more workspace than the allocation-free entry point's "
                   "static scratch holds";
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
    c->ws = nullptr;
    int rc = device_info(device, c->info);
    if (rc == SV_OK) {
        // The draw pass splits a request over workgroups only when the batch
        // has fewer requests than the GPU has CUs.
        const int mb = max_batch < kLaunchBatch ? max_batch : kLaunchBatch;
        c->lay = ws_layout(mb, max_k, c->C, mb < c->info.cus ? mb : c->info.cus);
        void* w = nullptr;
        if (hipMalloc(&w, c->lay.total) != hipSuccess) {
            rc = SV_ERR_NOMEM;
        } else {
            c->ws = static_cast<unsigned char*>(w);
            if (hipMemset(c->ws, 0, c->lay.total) != hipSuccess ||
                hipDeviceSynchronize() != hipSuccess) {
                rc = SV_ERR_HIP;
            }
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

int spec_verify_run_ex(spec_verify_ctx* ctx, const void* target_logits, const void* draft_logits,
                       const int32_t* draft_tokens, const int32_t* budgets, int B, int K,
                       float temperature, uint64_t seed, int64_t request_base,
                       int32_t* out_tokens, int32_t* out_num_accepted, float* out_p_draft,
                       float* out_q_draft, void* stream) {
    if (!ctx || ctx->magic != kMagic) return SV_ERR_STATE;
    const int rc = spec_verify_check_args(ctx->max_batch, ctx->max_k, ctx->vocab, ctx->dtype,
                                          target_logits, draft_logits, draft_tokens, budgets, B,
                                          K, temperature, out_tokens, out_num_accepted,
                                          out_p_draft, out_q_draft);
    if (rc != SV_OK) return rc;
    if (request_base < 0 || request_base > (int64_t)0xFFFFFFFFll - B) return SV_ERR_ARG;
    if (B == 0) return SV_OK;
    int prev = -1;
    if (hipGetDevice(&prev) != hipSuccess) return SV_ERR_HIP;
    if (prev != ctx->device && hipSetDevice(ctx->device) != hipSuccess) return SV_ERR_HIP;
    RunArgs a{target_logits, draft_logits, draft_tokens, budgets, B, K, temperature, seed,
              (uint32_t)request_base, out_tokens, out_num_accepted, out_p_draft, out_q_draft};
    const int r = run_batches(ctx->info, ctx, ctx->vocab, ctx->dtype, ctx->ws, ctx->lay,
                              ctx->calls, reinterpret_cast<unsigned*>(ctx->ws + ctx->lay.status),
                              a, static_cast<hipStream_t>(stream));
    if (prev != ctx->device) (void)hipSetDevice(prev);
    return r;
}

int spec_verify_run(spec_verify_ctx* ctx, const void* target_logits, const void* draft_logits,
                    const int32_t* draft_tokens, const int32_t* budgets, int B, int K,
                    float temperature, uint64_t seed, int32_t* out_tokens,
                    int32_t* out_num_accepted, float* out_p_draft, float* out_q_draft,
                    void* stream) {
    return spec_verify_run_ex(ctx, target_logits, draft_logits, draft_tokens, budgets, B, K,
                              temperature, seed, 0, out_tokens, out_num_accepted, out_p_draft,
                              out_q_draft, stream);
}

int spec_verify_run_noalloc(int vocab, int dtype, const void* target_logits,
                            const void* draft_logits, const int32_t* draft_tokens,
                            const int32_t* budgets, int B, int K, float temperature,
                            uint64_t seed, int64_t request_base, int32_t* out_tokens,
                            int32_t* out_num_accepted, float* out_p_draft, float* out_q_draft,
                            uint32_t* out_status, void* stream) {
    const int mb = B < 1 ? 1 : (B > SV_MAX_BATCH ? SV_MAX_BATCH : B);
    const int rc = spec_verify_check_args(mb, K < 0 ? 0 : K, vocab, dtype, target_logits,
                                          draft_logits, draft_tokens, budgets, B, K,
                                          temperature, out_tokens, out_num_accepted,
                                          out_p_draft, out_q_draft);
    if (rc != SV_OK) return rc;
    if (request_base < 0 || request_base > (int64_t)0xFFFFFFFFll - B) return SV_ERR_ARG;
    if (out_status && !aligned_to(out_status, 4)) return SV_ERR_ALIGN;
    if (B == 0) return SV_OK;
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess) return SV_ERR_HIP;
    if (dev < 0 || dev >= kMaxDevices) return SV_ERR_ARG;
    std::lock_guard<std::mutex> lock(g_noalloc_mu);
    NoallocDevice& nd = g_noalloc[dev];
    if (!nd.ready) {
        // Once per device, with the device current: the device address of
        // this device's copy of `scratch`.
        void* ptr = nullptr;
        if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)) != hipSuccess || !ptr) {
            return SV_ERR_HIP;
        }
        if (device_info(dev, nd.info) != SV_OK) return SV_ERR_HIP;
        nd.ptr = static_cast<unsigned char*>(ptr);
        nd.calls = 0;
        nd.ready = true;
    }
    const int lb = B < kLaunchBatch ? B : kLaunchBatch;
    const int C = chunks_for(vocab, dtype);
    const WsLayout L = ws_layout(lb, K, C, lb < nd.info.cus ? lb : nd.info.cus);
    if (L.total > (size_t)SV_NOALLOC_SCRATCH_BYTES) return SV_ERR_TOO_BIG;
    hipStream_t s = static_cast<hipStream_t>(stream);
    unsigned* req = reinterpret_cast<unsigned*>(nd.ptr + L.req);
    unsigned* dcnt = reinterpret_cast<unsigned*>(nd.ptr + L.dcnt);
    hipLaunchKernelGGL(clear_words_kernel, dim3(8), dim3(256), 0, s,
                       reinterpret_cast<unsigned*>(nd.ptr + L.team), (int)L.teams, req,
                       (int)((L.req_end - L.req) / 4), dcnt, (int)((L.dcnt_end - L.dcnt) / 4),
                       reinterpret_cast<unsigned*>(nd.ptr + L.status + 64), out_status);
    if (hipGetLastError() != hipSuccess) return SV_ERR_HIP;
    unsigned* status = out_status ? out_status : reinterpret_cast<unsigned*>(nd.ptr + L.status);
    RunArgs a{target_logits, draft_logits, draft_tokens, budgets, B, K, temperature, seed,
              (uint32_t)request_base, out_tokens, out_num_accepted, out_p_draft, out_q_draft};
    return run_batches(nd.info, nullptr, vocab, dtype, nd.ptr, L, nd.calls, status, a, s);
}

int spec_verify_status(spec_verify_ctx* ctx, uint32_t* flags) {
    if (!ctx || ctx->magic != kMagic) return SV_ERR_STATE;
    if (!flags) return SV_ERR_NULL;
    int prev = -1;
    if (hipGetDevice(&prev) != hipSuccess) return SV_ERR_HIP;
    if (prev != ctx->device && hipSetDevice(ctx->device) != hipSuccess) return SV_ERR_HIP;
    int rc = SV_OK;
    unsigned v = 0;
    unsigned* status = reinterpret_cast<unsigned*>(ctx->ws + ctx->lay.status);
    if (hipDeviceSynchronize() != hipSuccess ||
        hipMemcpy(&v, status, sizeof(v), hipMemcpyDeviceToHost) != hipSuccess ||
        hipMemset(status, 0, sizeof(unsigned)) != hipSuccess ||
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

int spec_verify_timing(spec_verify_ctx* ctx, int enable) {
    if (!ctx || ctx->magic != kMagic) return SV_ERR_STATE;
    int prev = -1;
    if (hipGetDevice(&prev) != hipSuccess) return SV_ERR_HIP;
    if (prev != ctx->device && hipSetDevice(ctx->device) != hipSuccess) return SV_ERR_HIP;
    int rc = SV_OK;
    if (!enable && !ctx->timed.empty()) {
        for (const auto& t : ctx->timed) {
            if (hipEventSynchronize(t.end) != hipSuccess) rc = SV_ERR_HIP;
            ctx->event_pool.push_back(t.start);
            ctx->event_pool.push_back(t.end);
        }
        ctx->timed.clear();
    }
    ctx->timing = enable != 0;
    if (prev != ctx->device) (void)hipSetDevice(prev);
    return rc;
}

int spec_verify_timing_read(spec_verify_ctx* ctx, int* counts, double* total_ms) {
    if (!ctx || ctx->magic != kMagic) return SV_ERR_STATE;
    if (!counts || !total_ms) return SV_ERR_NULL;
    int prev = -1;
    if (hipGetDevice(&prev) != hipSuccess) return SV_ERR_HIP;
    if (prev != ctx->device && hipSetDevice(ctx->device) != hipSuccess) return SV_ERR_HIP;
    int rc = SV_OK;
    counts[0] = counts[1] = 0;
    total_ms[0] = total_ms[1] = 0.0;
    for (const auto& t : ctx->timed) {
        float ms = 0.0f;
        if (hipEventSynchronize(t.end) != hipSuccess ||
            hipEventElapsedTime(&ms, t.start, t.end) != hipSuccess) {
            rc = SV_ERR_HIP;
        } else {
            counts[t.pass] += 1;
            total_ms[t.pass] += (double)ms;
        }
        ctx->event_pool.push_back(t.start);
        ctx->event_pool.push_back(t.end);
    }
    ctx->timed.clear();
    if (prev != ctx->device) (void)hipSetDevice(prev);
    return rc;
}

void spec_verify_free(spec_verify_ctx* ctx) {
    if (!ctx || ctx->magic != kMagic) return;
    int prev = -1;
    (void)hipGetDevice(&prev);
    if (prev != ctx->device) (void)hipSetDevice(ctx->device);
    (void)hipDeviceSynchronize();
    for (hipEvent_t e : ctx->event_pool) (void)hipEventDestroy(e);
    for (const auto& t : ctx->timed) {
        (void)hipEventDestroy(t.start);
        (void)hipEventDestroy(t.end);
    }
    if (ctx->ws) (void)hipFree(ctx->ws);
    if (prev != ctx->device && prev >= 0) (void)hipSetDevice(prev);
    ctx->magic = 0;
    ctx->ws = nullptr;
    delete ctx;
}

}  // extern "C"
