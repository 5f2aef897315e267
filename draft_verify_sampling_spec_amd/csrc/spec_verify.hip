// spec_verify.hip -- batched draft verification for MI355X (gfx950, wave64).
//
// What is computed: "Speculative decoding becomes standard: DSpark and
// multi-token drafters", section "Why draft-and-verify does not change the
// output" (greedy keep-while-agreeing rule, paragraph 1; the sampled
// min(1, p/q) acceptance with residual resampling, paragraph 2), with the
// per-request verify budgets of section "What DSpark adds", paragraph 2.
// The ABI and its conventions are documented in include/spec_verify.h.
//
// Design (one fused, persistent kernel per call):
//  * Work unit = one vocabulary chunk of one logit row of one request. Every
//    chunk has the same size, so units balance perfectly; units are numbered
//    request-major (target row 0, drafter row 0, target row 1, ...), and
//    workgroups pull them from eight queues, one per XCD (workgroup w starts
//    on queue w % 8, the XCD the dispatcher places it on, and steals from the
//    others once its own is empty).
//  * A unit's rows are streamed with 16-byte loads, every load of the unit in
//    flight at once (8 per lane), reduced in registers: row max, then the sum
//    of 2^((z - max) * log2(e)/T) (sampled) or the (max, lowest index) pair
//    (greedy). The chunk's partial result goes to the workspace.
//  * Each request counts its finished units. The workgroup that finishes the
//    last one (release/acquire on the counter, no waiting anywhere) merges
//    the partials, takes the accept decisions and the first-reject scan in one
//    wave, then draws the residual / bonus token with the whole workgroup: a
//    pass computing per-tile masses into LDS, a scan over tiles, and an
//    element-level scan of the one tile holding the threshold. Because the
//    request's units were processed moments earlier, the re-read row pair is
//    served by the caches rather than HBM.
//  * Counters clean themselves: the last arriver of a request zeroes its
//    counter, the last workgroup to exit zeroes the queues.

#include <hip/hip_runtime.h>

#include <climits>
#include <cmath>
#include <cstdint>
#include <cstring>

#include "spec_verify.h"

namespace {

constexpr int kThreads = 256;                 // workgroup size (4 waves)
constexpr int kWaves = kThreads / 64;
constexpr int kGroupsPerThread = 8;           // 16-byte loads per lane per unit
constexpr int kTileElems = kThreads * 8;      // elements per sampling tile
constexpr int kTilesPerPass = 4;              // tiles whose loads are in flight together
constexpr int kNumQueues = 8;                 // one per XCD
constexpr int kCounterStride = 32;            // 128 bytes between counters
constexpr int kExitCounter = kNumQueues;      // index (in strides) of the exit counter
constexpr int kCounterWords = (kNumQueues + 1) * kCounterStride;

// Philox4x32 constants (Salmon et al., SC'11): round multipliers and the key
// increments applied between rounds.
constexpr uint32_t kPhiloxM0 = 0xD2511F53u;
constexpr uint32_t kPhiloxM1 = 0xCD9E8D57u;
constexpr uint32_t kPhiloxW0 = 0x9E3779B9u;
constexpr uint32_t kPhiloxW1 = 0xBB67AE85u;

constexpr double kLog2e = 1.4426950408889634073599246810019;

// Partial result of one chunk of one row.
//   sampled: m = chunk max, s = sum over the chunk of 2^((z - m) * c)
//   greedy:  m = chunk max, idx = lowest index attaining it
struct Partial {
    float m;
    int idx;
    double s;
};
static_assert(sizeof(Partial) == 16, "Partial layout");

struct Params {
    const void* target;       // [B, K+1, V]
    const void* draft;        // [B, K, V] (sampled mode)
    const int32_t* tokens;    // [B, K]
    const int32_t* budgets;   // [B]
    int32_t* out_tokens;      // [B, K+1]
    int32_t* out_nacc;        // [B]
    float* out_p;             // [B, K] or null
    float* out_q;             // [B, K] or null
    Partial* partials;        // [B, slots, C]
    int* arrive;              // [B]
    unsigned* counters;       // kCounterWords
    unsigned* status;         // 1 word
    int B, K, V;
    int C;                    // chunks per row
    int CE;                   // elements per chunk (a multiple of the 16-byte group)
    int slots;                // rows per request held in the partial layout (2K+1 or K+1)
    int tiles;                // ceil(V / kTileElems)
    float c32;                // log2(e) / T
    double c64;
    uint32_t key0, key1;
};

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

// Load the group of elements [e, e + W) of a row; elements at or beyond `n`
// read as -inf. `vec_ok` says 16-byte loads are legal for this row segment.
template <typename E>
__device__ __forceinline__ uint4 load_group(const E* base, int e, int n, bool vec_ok) {
    constexpr int W = Elem<E>::W;
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

// --------------------------------------------------------- shared memory --

struct Shared {
    float red_f[kWaves];
    int red_i[kWaves];
    double red_d[kWaves];
    int unit;               // next unit of this workgroup (-1: none)
    int last;               // this workgroup finished the last unit of a request
    int last_b;
    // decision -> sampler hand-off
    int j, k, mode;         // mode 0: residual, 1: bonus (target row only)
    float mt, md;
    float inv_st, inv_sd;
    double u;
    double R;
    int tile_star;
    double base;
};

// Units per request for budget k.
__device__ __forceinline__ int units_of(int k, int C, bool greedy) {
    return (greedy ? (k + 1) : (2 * k + 1)) * C;
}

// ------------------------------------------------------------ work queue --

// Thread 0 only. `q` counts the queues this workgroup found empty.
__device__ int fetch_unit(unsigned* counters, int U, int home, int& q) {
    while (q < kNumQueues) {
        const int qi = (home + q) % kNumQueues;
        const int lo = (int)(((long long)U * qi) / kNumQueues);
        const int hi = (int)(((long long)U * (qi + 1)) / kNumQueues);
        const unsigned idx = __hip_atomic_fetch_add(&counters[qi * kCounterStride], 1u,
                                                    __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        if ((long long)idx < (long long)(hi - lo)) return lo + (int)idx;
        ++q;
    }
    return -1;
}

// -------------------------------------------------------- sampling pass --

// Unnormalised-free residual (or bonus) mass of the 8 elements starting at e.
template <typename E>
__device__ __forceinline__ void tile_mass(const E* rt, const E* rd, int e, int V, bool vt,
                                          bool vd, float mt, float inv_st, float md,
                                          float inv_sd, float c, float r[8]) {
    constexpr int W = Elem<E>::W;
    #pragma unroll
    for (int h = 0; h < 8 / W; ++h) {
        const uint4 gt = load_group<E>(rt, e + h * W, V, vt);
        float pt[W];
        #pragma unroll
        for (int k = 0; k < W; ++k) pt[k] = fast_exp2((Elem<E>::at(gt, k) - mt) * c) * inv_st;
        if (rd != nullptr) {
            const uint4 gd = load_group<E>(rd, e + h * W, V, vd);
            #pragma unroll
            for (int k = 0; k < W; ++k) {
                const float qd = fast_exp2((Elem<E>::at(gd, k) - md) * c) * inv_sd;
                r[h * W + k] = fmaxf(0.0f, pt[k] - qd);
            }
        } else {
            #pragma unroll
            for (int k = 0; k < W; ++k) r[h * W + k] = pt[k];
        }
    }
}

// Inverse-CDF draw from the mass of the row (pair) described in `sh`:
// y = smallest v with (running mass up to v) > u * (total mass), zero-mass
// tokens excluded. Whole workgroup; returns y in every thread.
template <typename E>
__device__ int sample_row(const Params& P, Shared& sh, double* tile_sums, const E* rt,
                          const E* rd) {
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int V = P.V, tiles = P.tiles;
    const bool vt = (reinterpret_cast<uintptr_t>(rt) & 15) == 0;
    const bool vd = rd != nullptr && (reinterpret_cast<uintptr_t>(rd) & 15) == 0;
    const float mt = sh.mt, md = sh.md, inv_st = sh.inv_st, inv_sd = sh.inv_sd;
    const float c = P.c32;

    // Pass 1: mass of every (tile, wave) segment.
    for (int t0 = 0; t0 < tiles; t0 += kTilesPerPass) {
        float r[kTilesPerPass][8];
        #pragma unroll
        for (int a = 0; a < kTilesPerPass; ++a) {
            const int e = (t0 + a) * kTileElems + tid * 8;
            if (t0 + a < tiles) {
                tile_mass<E>(rt, rd, e, V, vt, vd, mt, inv_st, md, inv_sd, c, r[a]);
            }
        }
        #pragma unroll
        for (int a = 0; a < kTilesPerPass; ++a) {
            if (t0 + a < tiles) {
                float ls = 0.0f;
                #pragma unroll
                for (int k = 0; k < 8; ++k) ls += r[a][k];
                const double ws = wave_sum((double)ls);
                if (lane == 0) tile_sums[(t0 + a) * kWaves + wave] = ws;
            }
        }
    }
    __syncthreads();

    // Pass 2 (wave 0): total mass, threshold, and the tile holding it.
    if (wave == 0) {
        const int per = (tiles + 63) / 64;
        const int a0 = min(lane * per, tiles), a1 = min(a0 + per, tiles);
        double acc = 0.0;
        for (int t = a0; t < a1; ++t) {
            const double* ts = tile_sums + t * kWaves;
            acc += ((ts[0] + ts[1]) + ts[2]) + ts[3];
        }
        const double incl = wave_incl_scan(acc, lane);
        const double prev = __shfl_up(incl, 1, 64);
        const double R = __shfl(incl, 63, 64);
        const double thr = sh.u * R;
        const unsigned long long hit = __ballot(incl > thr);
        const int lane_star = hit ? (__ffsll((long long)hit) - 1) : 63;
        if (lane == lane_star) {
            double base = lane ? prev : 0.0;
            int found = -1, last_pos = -1;
            double base_last = 0.0;
            for (int t = a0; t < a1; ++t) {
                const double* ts = tile_sums + t * kWaves;
                const double tt = ((ts[0] + ts[1]) + ts[2]) + ts[3];
                if (tt > 0.0) {
                    last_pos = t;
                    base_last = base;
                }
                if (tt > 0.0 && base + tt > thr) {
                    found = t;
                    break;
                }
                base += tt;
            }
            if (found < 0) {          // rounding left the crossing past this lane's tiles
                found = last_pos;
                base = base_last;
            }
            sh.tile_star = found;
            sh.base = base;
            sh.R = R;
        }
    }
    __syncthreads();
    if (!(sh.R > 0.0) || sh.tile_star < 0) return -1;   // no mass at all

    // Pass 3: element-level scan of the chosen tile.
    const int ts = sh.tile_star;
    const int e = ts * kTileElems + tid * 8;
    float r[8];
    tile_mass<E>(rt, rd, e, V, vt, vd, mt, inv_st, md, inv_sd, c, r);
    double pre[8];
    double run = 0.0;
    #pragma unroll
    for (int k = 0; k < 8; ++k) {
        run += (double)r[k];
        pre[k] = run;
    }
    // Block exclusive scan of the per-thread totals.
    double incl = wave_incl_scan(run, lane);
    if (lane == 63) sh.red_d[wave] = incl;
    __syncthreads();
    double excl = incl - run;
    {
        // Use the exact lane-exclusive value rather than incl - run.
        const double up = __shfl_up(incl, 1, 64);
        excl = lane ? up : 0.0;
    }
    for (int w = 0; w < wave; ++w) excl += sh.red_d[w];
    const double thr = sh.u * sh.R - sh.base;
    int cand = INT_MAX, last_pos = -1;
    #pragma unroll
    for (int k = 0; k < 8; ++k) {
        if (r[k] > 0.0f) {
            last_pos = e + k;
            if (cand == INT_MAX && excl + pre[k] > thr) cand = e + k;
        }
    }
    // Block min of candidates, block max of last positive index.
    #pragma unroll
    for (int off = 32; off > 0; off >>= 1) {
        cand = min(cand, __shfl_xor(cand, off, 64));
        last_pos = max(last_pos, __shfl_xor(last_pos, off, 64));
    }
    __syncthreads();
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

// ---------------------------------------------------------- main kernel --

template <typename E, bool kGreedy>
__global__ __launch_bounds__(kThreads) void verify_kernel(Params P) {
    extern __shared__ __align__(16) unsigned char dyn_smem[];
    __shared__ Shared sh;
    // Dynamic LDS: per-(tile, wave) sampling masses, then request unit offsets.
    double* tile_sums = reinterpret_cast<double*>(dyn_smem);
    int* off = reinterpret_cast<int*>(dyn_smem + (kGreedy ? 0 : (size_t)P.tiles * kWaves * 8));

    constexpr int W = Elem<E>::W;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int B = P.B, K = P.K, V = P.V, C = P.C;

    // Prologue: every workgroup scans the budgets into unit offsets.
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
            local += units_of(k, C, kGreedy);
        }
        if (bad && blockIdx.x == 0) atomicOr(P.status, SV_FLAG_BAD_BUDGET);
        // Block exclusive scan of `local`.
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
            run += units_of(k, C, kGreedy);
        }
        if (tid == kThreads - 1) off[B] = run;
        __syncthreads();
    }
    const int U = off[B];
    const int home = blockIdx.x % kNumQueues;
    int qpos = 0;                                   // thread 0's queue cursor

    if (tid == 0) sh.unit = fetch_unit(P.counters, U, home, qpos);
    __syncthreads();

    const E* target = static_cast<const E*>(P.target);
    const E* draft = static_cast<const E*>(P.draft);

    for (;;) {
        const int u = sh.unit;
        if (u < 0) break;
        // Decode the unit: request b (largest b with off[b] <= u), row slot, chunk.
        int lo = 0, hi = B;
        while (hi - lo > 1) {
            const int mid = (lo + hi) >> 1;
            if (off[mid] <= u) lo = mid; else hi = mid;
        }
        const int b = lo;
        const int local = u - off[b];
        const int slot = local / C;
        const int chunk = local - slot * C;
        const int n_units = off[b + 1] - off[b];
        const E* row;
        if (kGreedy) {
            row = target + ((size_t)b * (K + 1) + slot) * (size_t)V;
        } else if (slot & 1) {
            row = draft + ((size_t)b * K + (slot >> 1)) * (size_t)V;
        } else {
            row = target + ((size_t)b * (K + 1) + (slot >> 1)) * (size_t)V;
        }
        const int e0 = chunk * P.CE;
        const int n = min(P.CE, V - e0);
        const E* base = row + e0;
        const bool vec_ok = (reinterpret_cast<uintptr_t>(base) & 15) == 0;
        const int ngroups = (n + W - 1) / W;

        int next = -1;
        if (tid == 0) next = fetch_unit(P.counters, U, home, qpos);

        uint4 g[kGroupsPerThread];
        #pragma unroll
        for (int j = 0; j < kGroupsPerThread; ++j) {
            const int gi = tid + j * kThreads;
            if (gi < ngroups) {
                g[j] = load_group<E>(base, gi * W, n, vec_ok);
            } else {
                g[j] = make_uint4(Elem<E>::kNegInfWord, Elem<E>::kNegInfWord,
                                  Elem<E>::kNegInfWord, Elem<E>::kNegInfWord);
            }
        }

        Partial part;
        if (kGreedy) {
            float bv = -INFINITY;
            int bi = INT_MAX;
            #pragma unroll
            for (int j = 0; j < kGroupsPerThread; ++j) {
                #pragma unroll
                for (int k = 0; k < W; ++k) {
                    const float v = Elem<E>::at(g[j], k);
                    const int idx = e0 + (tid + j * kThreads) * W + k;
                    if (v > bv) {           // groups and lanes go up in index order
                        bv = v;
                        bi = idx;
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
                sh.red_f[wave] = bv;
                sh.red_i[wave] = bi;
            }
            __syncthreads();
            if (tid == 0) {
                for (int w = 1; w < kWaves; ++w) {
                    if (better_arg(sh.red_f[w], sh.red_i[w], bv, bi)) {
                        bv = sh.red_f[w];
                        bi = sh.red_i[w];
                    }
                }
                part.m = bv;
                part.idx = bi;
                part.s = 0.0;
            }
        } else {
            float m = -INFINITY;
            #pragma unroll
            for (int j = 0; j < kGroupsPerThread; ++j) {
                #pragma unroll
                for (int k = 0; k < W; ++k) m = fmaxf(m, Elem<E>::at(g[j], k));
            }
            m = wave_max(m);
            if (lane == 0) sh.red_f[wave] = m;
            __syncthreads();
            float M = sh.red_f[0];
            #pragma unroll
            for (int w = 1; w < kWaves; ++w) M = fmaxf(M, sh.red_f[w]);
            float ls = 0.0f;
            if (M != -INFINITY) {
                const float c = P.c32;
                #pragma unroll
                for (int j = 0; j < kGroupsPerThread; ++j) {
                    float e[W];
                    #pragma unroll
                    for (int k = 0; k < W; ++k) e[k] = fast_exp2((Elem<E>::at(g[j], k) - M) * c);
                    // pairwise sum of the group
                    #pragma unroll
                    for (int h = W / 2; h > 0; h >>= 1) {
                        #pragma unroll
                        for (int k = 0; k < h; ++k) e[k] += e[k + h];
                    }
                    ls += e[0];
                }
            }
            const double ws = wave_sum((double)ls);
            if (lane == 0) sh.red_d[wave] = ws;
            __syncthreads();
            if (tid == 0) {
                part.m = M;
                part.idx = 0;
                part.s = ((sh.red_d[0] + sh.red_d[1]) + sh.red_d[2]) + sh.red_d[3];
            }
        }

        if (tid == 0) {
            P.partials[((size_t)b * P.slots + slot) * C + chunk] = part;
            const int old = __hip_atomic_fetch_add(&P.arrive[b], 1, __ATOMIC_RELEASE,
                                                   __HIP_MEMORY_SCOPE_AGENT);
            const bool last = old == n_units - 1;
            if (last) {
                __hip_atomic_store(&P.arrive[b], 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            }
            sh.last = last;
            sh.last_b = b;
            sh.unit = next;
        }
        __syncthreads();

        if (sh.last) {
            // This workgroup finished request b: decide and sample.
            __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
            const int k = kGreedy ? n_units / C - 1 : (n_units / C - 1) / 2;
            if (wave == 0) {
                const int i = lane;
                bool accept = true;          // lanes beyond the budget never reject
                int best = 0;
                double mt = 0.0, st = 1.0, md = 0.0, sd = 1.0;
                if (i <= k) {
                    const Partial* pt = P.partials + ((size_t)b * P.slots + (kGreedy ? i : 2 * i)) * C;
                    if (kGreedy) {
                        float bv = pt[0].m;
                        int bi = pt[0].idx;
                        for (int cc = 1; cc < C; ++cc) {
                            if (better_arg(pt[cc].m, pt[cc].idx, bv, bi)) {
                                bv = pt[cc].m;
                                bi = pt[cc].idx;
                            }
                        }
                        best = bi == INT_MAX ? 0 : bi;      // an all -inf row: index 0
                    } else {
                        float M = pt[0].m;
                        for (int cc = 1; cc < C; ++cc) M = fmaxf(M, pt[cc].m);
                        double S = 0.0;
                        for (int cc = 0; cc < C; ++cc) {
                            if (pt[cc].s > 0.0) S += pt[cc].s * exp2(((double)pt[cc].m - (double)M) * P.c64);
                        }
                        mt = M;
                        st = S;
                        if (i < k) {
                            const Partial* pd = P.partials + ((size_t)b * P.slots + 2 * i + 1) * C;
                            float Md = pd[0].m;
                            for (int cc = 1; cc < C; ++cc) Md = fmaxf(Md, pd[cc].m);
                            double Sd = 0.0;
                            for (int cc = 0; cc < C; ++cc) {
                                if (pd[cc].s > 0.0) Sd += pd[cc].s * exp2(((double)pd[cc].m - (double)Md) * P.c64);
                            }
                            md = Md;
                            sd = Sd;
                        }
                    }
                }
                if (i < k) {
                    const int x = P.tokens[(size_t)b * K + i];
                    const bool valid = x >= 0 && x < V;
                    if (!valid) atomicOr(P.status, SV_FLAG_BAD_TOKEN);
                    if (kGreedy) {
                        accept = valid && x == best;
                    } else {
                        double px = 0.0, qx = 0.0;
                        if (valid) {
                            const float zt = Elem<E>::one(target + ((size_t)b * (K + 1) + i) * (size_t)V + x);
                            const float zd = Elem<E>::one(draft + ((size_t)b * K + i) * (size_t)V + x);
                            px = exp2(((double)zt - mt) * P.c64) / st;
                            qx = exp2(((double)zd - md) * P.c64) / sd;
                        }
                        const uint4 rw = philox4x32_10((uint32_t)b, (uint32_t)i, 0u, 0u, P.key0, P.key1);
                        const double ua = word_to_uniform(rw.x);
                        accept = ua * qx < px;
                        if (P.out_p) P.out_p[(size_t)b * K + i] = (float)px;
                        if (P.out_q) P.out_q[(size_t)b * K + i] = (float)qx;
                    }
                } else if (i < K) {
                    if (P.out_p) P.out_p[(size_t)b * K + i] = NAN;
                    if (P.out_q) P.out_q[(size_t)b * K + i] = NAN;
                }
                if (kGreedy && i < K && i < k) {
                    if (P.out_p) P.out_p[(size_t)b * K + i] = NAN;
                    if (P.out_q) P.out_q[(size_t)b * K + i] = NAN;
                }
                const unsigned long long rej = __ballot(!accept);
                const int j = rej ? (__ffsll((long long)rej) - 1) : k;
                // Emitted tokens other than the drawn one.
                if (i <= K && i != j) {
                    int32_t v = -1;
                    if (i < j) v = P.tokens[(size_t)b * K + i];
                    P.out_tokens[(size_t)b * (K + 1) + i] = v;
                }
                if (i == 0) P.out_nacc[b] = j;
                if (kGreedy) {
                    const int yj = __shfl(best, j, 64);
                    if (i == 0) P.out_tokens[(size_t)b * (K + 1) + j] = yj;
                } else {
                    const double mtj = __shfl(mt, j, 64), stj = __shfl(st, j, 64);
                    const double mdj = __shfl(md, j, 64), sdj = __shfl(sd, j, 64);
                    if (i == 0) {
                        sh.j = j;
                        sh.k = k;
                        sh.mode = j < k ? 0 : 1;
                        sh.mt = (float)mtj;
                        sh.inv_st = (float)(1.0 / stj);
                        sh.md = (float)mdj;
                        sh.inv_sd = (float)(1.0 / sdj);
                        const uint4 rw = philox4x32_10((uint32_t)b, (uint32_t)j, 0u, 0u, P.key0, P.key1);
                        sh.u = word_to_uniform(rw.y);
                    }
                }
            }
            __syncthreads();
            if (!kGreedy) {
                const int j = sh.j;
                const E* rt = target + ((size_t)b * (K + 1) + j) * (size_t)V;
                const E* rd = sh.mode == 0 ? draft + ((size_t)b * K + j) * (size_t)V : nullptr;
                int y = sample_row<E>(P, sh, tile_sums, rt, rd);
                if (y < 0 && rd != nullptr) {
                    // The residual kept no mass (rounding only): draw from p_j.
                    y = sample_row<E>(P, sh, tile_sums, rt, nullptr);
                }
                if (tid == 0) P.out_tokens[(size_t)b * (K + 1) + j] = y < 0 ? 0 : y;
                __syncthreads();
            }
        }
    }

    // Exit: the last workgroup out resets the queues for the next call.
    if (tid == 0) {
        const unsigned old = __hip_atomic_fetch_add(&P.counters[kExitCounter * kCounterStride], 1u,
                                                    __ATOMIC_ACQ_REL, __HIP_MEMORY_SCOPE_AGENT);
        if (old == gridDim.x - 1) {
            for (int q = 0; q < kNumQueues; ++q) {
                __hip_atomic_store(&P.counters[q * kCounterStride], 0u, __ATOMIC_RELAXED,
                                   __HIP_MEMORY_SCOPE_AGENT);
            }
            __hip_atomic_store(&P.counters[kExitCounter * kCounterStride], 0u, __ATOMIC_RELAXED,
                               __HIP_MEMORY_SCOPE_AGENT);
        }
    }
}

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

int chunks_for(int vocab, int dtype) {
    const int w = dtype == SV_DTYPE_BF16 ? 8 : 4;
    const int per_unit = kThreads * kGroupsPerThread * w;
    return (vocab + per_unit - 1) / per_unit;
}

int chunk_elems(int vocab, int dtype, int C) {
    const int w = dtype == SV_DTYPE_BF16 ? 8 : 4;
    const int ce = (vocab + C - 1) / C;
    return (ce + w - 1) / w * w;
}

size_t dyn_smem_bytes(int B, int tiles, bool greedy) {
    return (greedy ? 0 : (size_t)tiles * kWaves * sizeof(double)) + (size_t)(B + 1) * sizeof(int);
}

}  // namespace

struct spec_verify_ctx {
    uint32_t magic;
    int device, max_batch, max_k, vocab, dtype;
    int C, CE, tiles;
    int cus;
    void* ws;
    Partial* partials;
    int* arrive;
    unsigned* counters;
    unsigned* status;
};

namespace {

template <typename E, bool G>
int occupancy_of(size_t smem) {
    int n = 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, verify_kernel<E, G>, kThreads, smem) !=
        hipSuccess) {
        return 1;
    }
    return n > 0 ? n : 1;
}

template <typename E, bool G>
hipError_t launch(const spec_verify_ctx* ctx, const Params& p, hipStream_t stream) {
    const size_t smem = dyn_smem_bytes(p.B, p.tiles, G);
    const int occ = occupancy_of<E, G>(smem);
    long long max_units = (long long)p.B * p.slots * p.C;
    long long grid = (long long)ctx->cus * occ;
    if (grid > max_units) grid = max_units;
    if (grid < 1) grid = 1;
    hipLaunchKernelGGL((verify_kernel<E, G>), dim3((unsigned)grid), dim3(kThreads), smem, stream,
                       p);
    return hipGetLastError();
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
    c->CE = chunk_elems(vocab, dtype, c->C);
    c->tiles = (vocab + kTileElems - 1) / kTileElems;
    int rc = SV_OK;
    if (hipDeviceGetAttribute(&c->cus, hipDeviceAttributeMultiprocessorCount, device) !=
        hipSuccess) {
        rc = SV_ERR_HIP;
    }
    const size_t slots = 2 * (size_t)max_k + 1;
    const size_t part_bytes = (size_t)max_batch * slots * c->C * sizeof(Partial);
    const size_t arrive_bytes = ((size_t)max_batch * sizeof(int) + 255) / 256 * 256;
    const size_t counter_bytes = (size_t)kCounterWords * sizeof(unsigned);
    const size_t total = part_bytes + arrive_bytes + counter_bytes + 256;
    if (rc == SV_OK && hipMalloc(&c->ws, total) != hipSuccess) {
        c->ws = nullptr;
        rc = SV_ERR_NOMEM;
    }
    if (rc == SV_OK) {
        unsigned char* w = static_cast<unsigned char*>(c->ws);
        c->partials = reinterpret_cast<Partial*>(w);
        c->arrive = reinterpret_cast<int*>(w + part_bytes);
        c->counters = reinterpret_cast<unsigned*>(w + part_bytes + arrive_bytes);
        c->status = reinterpret_cast<unsigned*>(w + part_bytes + arrive_bytes + counter_bytes);
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
    p.partials = ctx->partials;
    p.arrive = ctx->arrive;
    p.counters = ctx->counters;
    p.status = ctx->status;
    p.B = B;
    p.K = K;
    p.V = ctx->vocab;
    p.C = ctx->C;
    p.CE = ctx->CE;
    p.slots = greedy ? K + 1 : 2 * K + 1;
    p.tiles = ctx->tiles;
    p.c64 = greedy ? 0.0 : kLog2e / (double)temperature;
    p.c32 = (float)p.c64;
    p.key0 = (uint32_t)(seed & 0xFFFFFFFFu);
    p.key1 = (uint32_t)(seed >> 32);

    int prev = -1;
    if (hipGetDevice(&prev) != hipSuccess) return SV_ERR_HIP;
    if (prev != ctx->device && hipSetDevice(ctx->device) != hipSuccess) return SV_ERR_HIP;
    hipStream_t s = static_cast<hipStream_t>(stream);
    hipError_t e;
    if (ctx->dtype == SV_DTYPE_BF16) {
        e = greedy ? launch<uint16_t, true>(ctx, p, s) : launch<uint16_t, false>(ctx, p, s);
    } else {
        e = greedy ? launch<float, true>(ctx, p, s) : launch<float, false>(ctx, p, s);
    }
    if (prev != ctx->device) (void)hipSetDevice(prev);
    return e == hipSuccess ? SV_OK : SV_ERR_HIP;
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
