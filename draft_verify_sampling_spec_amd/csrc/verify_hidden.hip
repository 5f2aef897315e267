// verify_hidden.hip -- batched draft verification from hidden states through
// the shared output head, for MI355X (gfx950).
//
// What is computed: "Speculative decoding becomes standard: DSpark and
// multi-token drafters", section "What DSpark adds", paragraph 1 (the drafter
// reuses the target's output projection unchanged, so both models' logits for
// a position are that head applied to a hidden state), section "Why
// draft-and-verify does not change the output", paragraphs 1 and 2 (keep
// drafted tokens while the target agrees -- greedy: equal to its most likely
// token; sampled: u < min(1, p/q) -- then emit the target's own token drawn
// from the residual max(0, p - q), or one more token from the target when the
// whole budget survives), and section "What DSpark adds", paragraph 2 (ragged
// per-request budgets). The outputs are those of spec_verify_run on the
// logits z = h W^T, but the logits of the scored rows never reach memory.
//
// Design, five stream-ordered launches:
//   1. plan (one workgroup): clamps budgets, checks drafted tokens, and packs
//      the rows a request needs -- target rows 0..k_b, and in sampled mode
//      drafter rows 0..k_b-1 -- into a row map, with the row count left on
//      the device: every request's target rows first, then (from a multiple
//      of 8, so that no group of 8 packed rows mixes the two buffers) every
//      request's drafter rows;
//   2. the head product with the statistics epilogue over the packed rows
//      (max, exp-sum and drafted token's logit; greedy: first argmax), its
//      grid covering any count up to the batch's bound;
//   3. decide (a thread per request): p(x), q(x), the accept test with the
//      Philox uniforms, the first rejection; greedy outputs are final here;
//   4. sampled only: the head product once more for each request's draw rows
//      (target and drafter row j_b for a residual, target row k_b for a
//      bonus). When the many-row product takes them (at least 512 requests),
//      the rows are paired -- request b's target row at 16 (b / 8) + b % 8,
//      its drafter row 8 rows further -- and the product's epilogue turns
//      each pair's logits into draw masses per 32-column block (the residual
//      max(0, p - q) and p alone), so no logit reaches memory; otherwise
//      (every target row first, then from a multiple of 8 every drafter row)
//      it writes the rows' fp32 logits. Either way the logits are
//      bit-identical to the values the statistics were taken over when both
//      go through the many-row product (each accumulates in the same order);
//   5. sampled only: the inverse-CDF draw in vocabulary order, one workgroup
//      per request: from the block masses, the block where the running mass
//      crosses u R and that block's 32 logits recomputed by the same
//      matrix-core products (hv_pick_kernel); or, from the stored logits,
//      256-element block masses and a rescan of the crossing block
//      (hv_draw_kernel).

#include <hip/hip_runtime.h>

#include <climits>
#include <cmath>
#include <cstdint>

#include "head_gemm.h"
#include "philox_device.h"
#include "spec_verify.h"

namespace {

using svhead::HeadRows;
using svrng::philox4x32_10;
using svrng::word_to_uniform;

constexpr int kPlanThreads = 1024;
constexpr int kPlanWaves = kPlanThreads / 64;

using svhead::DrawDesc;
using svhead::DrawMass;
using svhead::kBonus;
using svhead::kNoDraw;
using svhead::kResidual;

// Workspace layout (byte offsets, each 256-aligned).
struct Layout {
    size_t rowmap, rowtok, off, offd, nrows, sm, ss, sz, sa, part, drawmap, desc, logits, total;
};

size_t up256(size_t x) { return (x + 255) & ~(size_t)255; }

// Packed rows at most: the target rows, up to 7 rows of padding, the
// drafter rows.
size_t packed_rows_max(int B, int K) { return (size_t)B * (2 * K + 1) + 7; }

// Draw rows: request b's target row at b, its drafter row at up8(B) + b
// (the logits path); or, paired (the mass path), request b's target row at
// 16 (b / 8) + b % 8 and its drafter row 8 rows further.
__host__ __device__ inline int draw_split(int B) { return (B + 7) & ~7; }
size_t draw_rows_for(int B) { return (size_t)draw_split(B) + (size_t)B; }
size_t paired_rows_for(int B) { return 2 * (size_t)draw_split(B); }
__host__ __device__ inline int paired_target_row(int b) { return 16 * (b >> 3) + (b & 7); }

// Blocks of 32 vocabulary columns (the mass path's draw masses).
__host__ __device__ inline int mass_blocks(int V) { return (V + 31) >> 5; }

Layout layout_for(int B, int K, int V) {
    const size_t rmax = packed_rows_max(B, K);
    Layout L{};
    size_t o = 0;
    auto take = [&](size_t bytes) {
        const size_t at = o;
        o += up256(bytes);
        return at;
    };
    L.rowmap = take(rmax * 4);
    L.rowtok = take(rmax * 4);
    L.off = take((size_t)B * 4);
    L.offd = take((size_t)B * 4);
    L.nrows = take(4);
    L.sm = take(rmax * 4);
    L.ss = take(rmax * 4);
    L.sz = take(rmax * 4);
    L.sa = take(rmax * 4);
    L.part = take(svhead::stats_workspace_bytes((int)rmax, V));
    L.drawmap = take(paired_rows_for(B) * 4);
    L.desc = take((size_t)B * sizeof(DrawDesc));
    // The draw rows' fp32 logits, or (the mass path) two arrays of B x
    // mass_blocks(V) x 2 fp64 half-block masses, which take less room.
    L.logits = take(draw_rows_for(B) * (size_t)V * 4);
    L.total = o;
    return L;
}

__device__ __forceinline__ int clamp_budget(int k, int K, unsigned& flags) {
    if (k < 0 || k > K) {
        flags |= SV_FLAG_BAD_BUDGET;
        return k < 0 ? 0 : K;
    }
    return k;
}

// Exclusive prefix over threads in thread order (each thread one count).
__device__ unsigned plan_exclusive(unsigned* wsum, unsigned v) {
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    unsigned incl = v;
    #pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
        const unsigned u = __shfl_up(incl, o, 64);
        if (lane >= o) incl += u;
    }
    if (lane == 63) wsum[wave] = incl;
    __syncthreads();
    unsigned base = 0;
    for (int w = 0; w < wave; ++w) base += wsum[w];
    return base + incl - v;
}

// Packed rows: request b's target rows 0..k (virtual row b (K+1) + i) at
// off[b] + i, all requests' target rows together from row 0; in sampled mode
// its drafter rows 0..k-1 (virtual row B (K+1) + b K + i) at offd[b] + i, all
// together from the first multiple of 8 after the target rows (the rows in
// between are rows of zeros, virtual row -1). Each carries the drafted token
// of its position (-1 for the target row k, for padding, and for a token
// outside [0, V), which is flagged).
__global__ __launch_bounds__(kPlanThreads) void hv_plan_kernel(
    const int32_t* __restrict__ budgets, const int32_t* __restrict__ tokens, int B, int K, int V,
    int greedy, int32_t* __restrict__ rowmap, int32_t* __restrict__ rowtok,
    int32_t* __restrict__ off, int32_t* __restrict__ offd, int32_t* __restrict__ nrows,
    int32_t* __restrict__ status) {
    __shared__ unsigned wsum[kPlanWaves];
    __shared__ unsigned flags_s, total_s;
    const int tid = threadIdx.x;
    if (tid == 0) flags_s = 0u;
    const int per = (B + kPlanThreads - 1) / kPlanThreads;
    const int b0 = min(tid * per, B), b1 = min(b0 + per, B);
    unsigned flags = 0u, cnt = 0u;
    for (int b = b0; b < b1; ++b) cnt += (unsigned)(clamp_budget(budgets[b], K, flags) + 1);
    const unsigned base_t = plan_exclusive(wsum, cnt);
    if (tid == kPlanThreads - 1) total_s = base_t + cnt;   // the target rows
    __syncthreads();
    const unsigned nt = total_s;
    const unsigned nt8 = (nt + 7u) & ~7u;
    unsigned ignore = 0u, cnt_d = 0u;
    for (int b = b0; b < b1; ++b) cnt_d += (unsigned)clamp_budget(budgets[b], K, ignore);
    const unsigned base_d = greedy ? 0u : nt8 + plan_exclusive(wsum, cnt_d);
    unsigned o = base_t, od = base_d;
    for (int b = b0; b < b1; ++b) {
        const int k = clamp_budget(budgets[b], K, ignore);
        off[b] = (int32_t)o;
        offd[b] = (int32_t)od;
        for (int i = 0; i <= k; ++i) {
            int x = -1;
            if (i < k) {
                x = tokens[(size_t)b * K + i];
                if (x < 0 || x >= V) {
                    flags |= SV_FLAG_BAD_TOKEN;
                    x = -1;
                }
            }
            rowmap[o + i] = b * (K + 1) + i;
            rowtok[o + i] = x;
            if (!greedy && i < k) {
                rowmap[od + i] = B * (K + 1) + b * K + i;
                rowtok[od + i] = x;
            }
        }
        o += (unsigned)(k + 1);
        od += (unsigned)k;
    }
    if (!greedy && tid < (int)(nt8 - nt)) {          // padding between the two parts
        rowmap[nt + tid] = -1;
        rowtok[nt + tid] = -1;
    }
    if (flags) atomicOr(&flags_s, flags);
    if (tid == kPlanThreads - 1) *nrows = (int32_t)(greedy ? nt : od);   // the last thread ends the packing
    __syncthreads();
    if (tid == 0 && status) *status = (int32_t)flags_s;
}

// One thread per request: the accept tests, the first rejection, the emitted
// drafted prefix; greedy also the target's token. Sampled requests leave a
// draw descriptor and their draw rows for the next two launches.
__global__ void hv_decide_kernel(const int32_t* __restrict__ budgets,
                                 const int32_t* __restrict__ tokens, int B, int K, int V,
                                 int greedy, double c64, uint32_t key0, uint32_t key1,
                                 const int32_t* __restrict__ off, const int32_t* __restrict__ offd,
                                 const float* __restrict__ sm,
                                 const float* __restrict__ ss, const float* __restrict__ sz,
                                 const int32_t* __restrict__ sa, int32_t* __restrict__ out_tokens,
                                 int32_t* __restrict__ out_n, float* __restrict__ out_p,
                                 float* __restrict__ out_q, int32_t* __restrict__ drawmap,
                                 DrawDesc* __restrict__ desc, int paired) {
    const int b = blockIdx.x * blockDim.x + threadIdx.x;
    // The draw rows' map: request b's target row at tb, its drafter row at db.
    const int tb = paired ? paired_target_row(b) : b;
    const int db = paired ? tb + 8 : draw_split(B) + b;
    if (b < draw_split(B) - B) {                       // padding rows
        const int bp = B + b;
        if (paired) {
            drawmap[paired_target_row(bp)] = -1;
            drawmap[paired_target_row(bp) + 8] = -1;
        } else {
            drawmap[bp] = -1;
        }
    }
    if (b >= B) return;
    unsigned ignore = 0u;
    const int k = clamp_budget(budgets[b], K, ignore);
    const int o = off[b], od = offd[b];
    int32_t* row = out_tokens + (size_t)b * (K + 1);
    int j = k;
    if (greedy) {
        for (int i = 0; i < k; ++i) {
            if (tokens[(size_t)b * K + i] != sa[o + i]) {
                j = i;
                break;
            }
        }
        for (int i = 0; i < j; ++i) row[i] = tokens[(size_t)b * K + i];
        row[j] = sa[o + j];
        for (int i = j + 1; i <= K; ++i) row[i] = -1;
        if (out_p) for (int i = 0; i < K; ++i) out_p[(size_t)b * K + i] = NAN;
        if (out_q) for (int i = 0; i < K; ++i) out_q[(size_t)b * K + i] = NAN;
        out_n[b] = j;
        DrawDesc d{};
        d.kind = kNoDraw;
        desc[b] = d;
        drawmap[tb] = -1;
        drawmap[db] = -1;
        return;
    }
    for (int i = 0; i < k; ++i) {
        const int x = tokens[(size_t)b * K + i];
        const bool valid = x >= 0 && x < V;
        const int rt = o + i, rd = od + i;
        double px = 0.0, qx = 0.0;
        if (valid) {
            px = exp2(((double)sz[rt] - (double)sm[rt]) * c64) / (double)ss[rt];
            qx = exp2(((double)sz[rd] - (double)sm[rd]) * c64) / (double)ss[rd];
        }
        const uint4 rw = philox4x32_10((uint32_t)b, (uint32_t)i, 0u, 0u, key0, key1);
        const bool accept = word_to_uniform(rw.x) * qx < px;
        if (out_p) out_p[(size_t)b * K + i] = (float)px;
        if (out_q) out_q[(size_t)b * K + i] = (float)qx;
        if (!accept && j == k) j = i;
    }
    for (int i = k; i < K; ++i) {
        if (out_p) out_p[(size_t)b * K + i] = NAN;
        if (out_q) out_q[(size_t)b * K + i] = NAN;
    }
    for (int i = 0; i < j; ++i) row[i] = tokens[(size_t)b * K + i];
    for (int i = j; i <= K; ++i) row[i] = -1;           // row[j] is the draw's
    out_n[b] = j;
    const uint4 rw = philox4x32_10((uint32_t)b, (uint32_t)j, 0u, 0u, key0, key1);
    DrawDesc d{};
    d.u = (float)word_to_uniform(rw.y);
    d.pos = j;
    d.mt = sm[o + j];
    d.st = ss[o + j];
    drawmap[tb] = b * (K + 1) + j;
    if (j < k) {
        d.kind = kResidual;
        d.md = sm[od + j];
        d.sd = ss[od + j];
        drawmap[db] = B * (K + 1) + b * K + j;
    } else {
        d.kind = kBonus;
        drawmap[db] = -1;
    }
    desc[b] = d;
}

// Running mass in vocabulary order over blocks of 256 elements: each lane
// holds 4 consecutive elements of a block (one 16-byte load per row), the
// block's mass is the fp64 wave sum of the lanes' fp32 sums, and the row's
// masses run block by block in fp64.
constexpr int kHvBlock = 256;
constexpr int kHvDrawWaves = 8;
constexpr int kHvDrawThreads = kHvDrawWaves * 64;
constexpr int kHvDrawSlots = 6;                    // blocks in flight per wave

__device__ __forceinline__ double hv_wave_sum(double v) {
    #pragma unroll
    for (int off = 32; off > 0; off >>= 1) v += __shfl_xor(v, off, 64);
    return v;
}

__device__ __forceinline__ double hv_wave_incl_scan(double v, int lane) {
    #pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
        const double o = __shfl_up(v, off, 64);
        if (lane >= off) v += o;
    }
    return v;
}

// Wave: the block where the running mass over blocks 0..n-1 first exceeds
// thr, and the mass before it (every lane); if rounding leaves no crossing,
// the last block with mass; -1 if no block has mass.
__device__ void hv_block_crossing(const double* m, int n, double thr, int& star, double& base) {
    const int lane = threadIdx.x & 63;
    const int per = (n + 63) / 64;
    const int a0 = min(lane * per, n), a1 = min(a0 + per, n);
    double acc = 0.0;
    for (int x = a0; x < a1; ++x) acc += m[x];
    const double incl = hv_wave_incl_scan(acc, lane);
    const double prev = __shfl_up(incl, 1, 64);
    const unsigned long long hit = __ballot(incl > thr);
    const unsigned long long pos = __ballot(acc > 0.0);
    const int ls = hit ? __ffsll((long long)hit) - 1 : (pos ? 63 - __clzll((long long)pos) : 63);
    int found = -1;
    double fb = 0.0;
    if (lane == ls) {
        double run = lane ? prev : 0.0;
        int last = -1;
        double run_last = 0.0;
        for (int x = a0; x < a1; ++x) {
            if (m[x] > 0.0) {
                last = x;
                run_last = run;
                if (run + m[x] > thr) {
                    found = x;
                    break;
                }
            }
            run += m[x];
        }
        if (found < 0) {
            found = last;
            run = run_last;
        }
        fb = run;
    }
    star = __shfl(found, ls, 64);
    base = __shfl(fb, ls, 64);
}

// The draw of one request (a workgroup of 8 waves). mass(v) = max(0, p(v) -
// q(v)) for a residual (p from the target row, q from the drafter row, each
// 2^((z - m) c) / S), p(v) for a bonus or when the residual has no mass. y is
// the smallest v whose running mass, in vocabulary order, exceeds u times the
// total; if rounding leaves no such v, the last v with positive mass. Every
// wave streams every eighth block of the row (or row pair) with
// kHvDrawSlots blocks in flight and leaves each block's mass in LDS; wave 0
// finds the block holding the threshold and scans its elements again.
template <bool kVec>
__global__ __launch_bounds__(kHvDrawThreads) __attribute__((amdgpu_waves_per_eu(4)))
void hv_draw_kernel(const float* __restrict__ logits, int K, int V, float c,
                    const DrawDesc* __restrict__ desc, int32_t* __restrict__ out_tokens) {
    extern __shared__ double blk[];                  // block masses [nb]
    __shared__ int star_s, resid_s;
    __shared__ double thr_s;
    const int b = blockIdx.x;
    const DrawDesc d = desc[b];
    if (d.kind == kNoDraw) return;                   // the whole workgroup
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const float* zt = logits + (size_t)b * V;
    const float* zd = logits + (size_t)(draw_split((int)gridDim.x) + b) * V;
    const int nb = (V + kHvBlock - 1) / kHvBlock;
    const int stride = kHvDrawSlots * kHvDrawWaves;
    const float ist = 1.0f / d.st;
    const float isd = d.kind == kResidual ? 1.0f / d.sd : 0.0f;

    // This lane's 4 elements of block x (past V: -inf, zero mass).
    auto load4 = [&](const float* row, int x) -> float4 {
        const int e = x * kHvBlock + lane * 4;
        if (kVec) {
            return e < V ? *reinterpret_cast<const float4*>(row + e)
                         : make_float4(-INFINITY, -INFINITY, -INFINITY, -INFINITY);
        }
        float4 r;
        r.x = e < V ? row[e] : -INFINITY;
        r.y = e + 1 < V ? row[e + 1] : -INFINITY;
        r.z = e + 2 < V ? row[e + 2] : -INFINITY;
        r.w = e + 3 < V ? row[e + 3] : -INFINITY;
        return r;
    };
    auto mass = [&](float t, float q, bool resid) -> float {
        const float p = __builtin_amdgcn_exp2f((t - d.mt) * c) * ist;
        if (!resid) return p;
        return fmaxf(p - __builtin_amdgcn_exp2f((q - d.md) * c) * isd, 0.0f);
    };
    auto mass4 = [&](const float4& t, const float4& q, bool resid, float (&r)[4]) {
        r[0] = mass(t.x, q.x, resid);
        r[1] = mass(t.y, q.y, resid);
        r[2] = mass(t.z, q.z, resid);
        r[3] = mass(t.w, q.w, resid);
    };

    for (int pass = 0; pass < 2; ++pass) {
        const bool resid = pass == 0 && d.kind == kResidual;
        float4 gt[kHvDrawSlots], gd[kHvDrawSlots];
        #pragma unroll
        for (int s = 0; s < kHvDrawSlots; ++s) {
            const int x = wave + s * kHvDrawWaves;
            if (x < nb) {
                gt[s] = load4(zt, x);
                if (resid) gd[s] = load4(zd, x);
            }
        }
        for (int xr = wave; xr < nb; xr += stride) {
            #pragma unroll
            for (int s = 0; s < kHvDrawSlots; ++s) {
                const int x = xr + s * kHvDrawWaves;
                if (x < nb) {
                    float r[4];
                    mass4(gt[s], gd[s], resid, r);
                    const double ws = hv_wave_sum((double)(((r[0] + r[1]) + r[2]) + r[3]));
                    if (lane == 0) blk[x] = ws;
                    if (x + stride < nb) {
                        gt[s] = load4(zt, x + stride);
                        if (resid) gd[s] = load4(zd, x + stride);
                    }
                }
            }
        }
        __syncthreads();
        if (wave == 0) {
            double total = 0.0;
            for (int x = lane; x < nb; x += 64) total += blk[x];
            total = hv_wave_sum(total);
            int star = -1;
            double base = 0.0;
            const double t = (double)d.u * total;
            if (total > 0.0) hv_block_crossing(blk, nb, t, star, base);
            if (lane == 0) {
                star_s = star;
                thr_s = t - base;
                resid_s = resid ? 1 : 0;
            }
        }
        __syncthreads();
        if (star_s >= 0 || !resid) break;               // no residual mass: from p
    }
    if (wave != 0) return;
    const int x = star_s;
    int y = 0;
    if (x >= 0) {
        const bool resid = resid_s != 0;
        const float4 t4 = load4(zt, x);
        const float4 q4 = resid ? load4(zd, x) : make_float4(0.0f, 0.0f, 0.0f, 0.0f);
        float r[4];
        mass4(t4, q4, resid, r);
        double pre[4];
        double run = 0.0;
        #pragma unroll
        for (int k = 0; k < 4; ++k) {
            run += (double)r[k];
            pre[k] = run;
        }
        const double incl = hv_wave_incl_scan(run, lane);
        const double up = __shfl_up(incl, 1, 64);
        const double excl = lane ? up : 0.0;
        const double tt = thr_s;
        const int e = x * kHvBlock + lane * 4;
        int cand = INT_MAX, last = -1;
        #pragma unroll
        for (int k = 0; k < 4; ++k) {
            if (r[k] > 0.0f) {
                last = e + k;
                if (cand == INT_MAX && excl + pre[k] > tt) cand = e + k;
            }
        }
        #pragma unroll
        for (int o = 32; o > 0; o >>= 1) {
            cand = min(cand, __shfl_xor(cand, o, 64));
            last = max(last, __shfl_xor(last, o, 64));
        }
        y = cand != INT_MAX ? cand : (last >= 0 ? last : 0);
    }
    if (lane == 0) out_tokens[(size_t)b * (K + 1) + d.pos] = y;
}

// The mass path's draw (one 4-wave workgroup per request), from the block
// masses of the paired product: the 32-column block where the running mass
// in vocabulary order first exceeds u times the total (the residual's, or
// p's for a bonus draw or a residual without mass), then that block's
// logits again -- the target row's and, for a residual, the drafter row's --
// from the same matrix-core products in the same order as the product's, so
// bit for bit the values its masses were taken over; then the first column
// whose running mass exceeds the rest of the threshold (if rounding leaves
// none, the last column with mass).
constexpr int kPickThreads = 256;

typedef float pk_f32x16 __attribute__((ext_vector_type(16)));
typedef __bf16 pk_bf16x8 __attribute__((ext_vector_type(8)));

// Dynamic LDS of hv_pick_kernel: the block masses, then the two hidden rows.
size_t pick_smem_bytes(int V, int H) { return (size_t)mass_blocks(V) * 8 + (size_t)4 * H; }
constexpr size_t kPickSmemMax = 64 * 1024;

__global__ __launch_bounds__(kPickThreads)
void hv_pick_kernel(const uint16_t* __restrict__ th, const uint16_t* __restrict__ dh,
                    const uint16_t* __restrict__ w, const int32_t* __restrict__ drawmap,
                    int a_rows, int K, int H, int V, float c, const DrawDesc* __restrict__ desc,
                    const double* __restrict__ mres, const double* __restrict__ mp,
                    int32_t* __restrict__ out_tokens) {
    extern __shared__ __align__(16) unsigned char pk_smem[];
    __shared__ int star_s, resid_s;
    __shared__ double thr_s;
    __shared__ float col_m[32];
    const int b = blockIdx.x;
    const DrawDesc d = desc[b];
    if (d.kind == kNoDraw) return;                   // the whole workgroup
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int nb = mass_blocks(V);
    double* blk = reinterpret_cast<double*>(pk_smem);
    uint16_t* hs = reinterpret_cast<uint16_t*>(pk_smem + (size_t)nb * 8);   // [2][H]
    const int tr = drawmap[paired_target_row(b)], dr = drawmap[paired_target_row(b) + 8];
    // The two hidden rows into LDS (zeros for a row that is not drawn from).
    for (int e = tid * 8; e < 2 * H; e += kPickThreads * 8) {
        const int row = e >= H, k = e - row * H;
        const uint16_t* src = nullptr;
        if (row == 0 && tr >= 0) src = th + (size_t)tr * H;
        if (row == 1 && d.kind == kResidual && dr >= 0) src = dh + (size_t)(dr - a_rows) * H;
        *reinterpret_cast<uint4*>(hs + e) = src ? *reinterpret_cast<const uint4*>(src + k)
                                                : make_uint4(0u, 0u, 0u, 0u);
    }
    for (int pass = 0; pass < 2; ++pass) {
        const bool resid = pass == 0 && d.kind == kResidual;
        // Each block's mass: the sum of its two halves.
        const double2* m = reinterpret_cast<const double2*>(resid ? mres : mp) + (size_t)b * nb;
        for (int x0 = tid; x0 < nb; x0 += 8 * kPickThreads) {
            double2 v[8];
            #pragma unroll
            for (int u = 0; u < 8; ++u) {
                v[u] = x0 + u * kPickThreads < nb ? m[x0 + u * kPickThreads] : make_double2(0.0, 0.0);
            }
            #pragma unroll
            for (int u = 0; u < 8; ++u) {
                if (x0 + u * kPickThreads < nb) blk[x0 + u * kPickThreads] = v[u].x + v[u].y;
            }
        }
        __syncthreads();
        if (wave == 0) {
            double total = 0.0;
            for (int x = lane; x < nb; x += 64) total += blk[x];
            total = hv_wave_sum(total);
            int star = -1;
            double base = 0.0;
            const double t = (double)d.u * total;
            if (total > 0.0) hv_block_crossing(blk, nb, t, star, base);
            if (lane == 0) {
                star_s = star;
                thr_s = t - base;
                resid_s = resid ? 1 : 0;
            }
        }
        __syncthreads();
        if (star_s >= 0 || !resid) break;               // no residual mass: from p
        __syncthreads();                                // blk is read again below
    }
    if (wave != 0) return;
    const int x = star_s;
    int y = 0;
    if (x >= 0) {
        const bool resid = resid_s != 0;
        // Vocabulary row v0 + lane % 32 as the first operand, hidden rows as
        // the second (slot 0 the target row, slot 8 the drafter row, zeros
        // elsewhere), this lane's 8 of each 16 of k: the product's layout.
        const int v0 = 32 * x;
        const int vr = v0 + (lane & 31);
        const int kh = 8 * (lane >> 5);
        const int slot = lane & 31;
        const uint16_t* wrow = w + (size_t)(vr < V ? vr : 0) * H;
        const uint16_t* hrow = slot == 0 ? hs : (slot == 8 ? hs + H : nullptr);
        const pk_bf16x8 zero8 = {};
        pk_f32x16 acc = {};
        constexpr int kDepth = 16;                      // groups of 16 of k in flight
        const int ng = H / 16;
        for (int g0 = 0; g0 < ng; g0 += kDepth) {
            pk_bf16x8 wa[kDepth];
            #pragma unroll
            for (int u = 0; u < kDepth; ++u) {
                const int g = g0 + u;
                wa[u] = (g < ng && vr < V)
                            ? *reinterpret_cast<const pk_bf16x8*>(wrow + 16 * g + kh) : zero8;
            }
            #pragma unroll
            for (int u = 0; u < kDepth; ++u) {
                const int g = g0 + u;
                if (g < ng) {
                    const pk_bf16x8 hb = hrow ? *reinterpret_cast<const pk_bf16x8*>(hrow + 16 * g + kh)
                                              : zero8;
                    acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(wa[u], hb, acc, 0, 0, 0);
                }
            }
        }
        // Lane l holds hidden slot l % 32 and 16 columns of the block: column
        // 8 (i / 4) + i % 4 + 4 (l / 32) for element i. Element masses as the
        // product's epilogue takes them.
        const float k = slot == 0 ? svhead::mass_offset(d.mt, d.st, c)
                                  : (resid && slot == 8 ? svhead::mass_offset(d.md, d.sd, c) : INFINITY);
        #pragma unroll
        for (int i = 0; i < 16; ++i) {
            const float e = __builtin_amdgcn_exp2f(__builtin_fmaf(acc[i], c, -k));
            const float q = __shfl_xor(e, 8, 64);
            const int col = 8 * (i >> 2) + (i & 3) + 4 * (lane >> 5);
            if (slot == 0) col_m[col] = v0 + col < V ? (resid ? fmaxf(e - q, 0.0f) : e) : 0.0f;
        }
        if (lane == 0) {
            const double tt = thr_s;
            double run = 0.0;
            int cand = -1, last = -1;
            for (int k2 = 0; k2 < 32; ++k2) {
                const float r = col_m[k2];
                if (r > 0.0f) {
                    last = v0 + k2;
                    run += (double)r;
                    if (cand < 0 && run > tt) cand = v0 + k2;
                }
            }
            y = cand >= 0 ? cand : (last >= 0 ? last : 0);
        }
    }
    if (lane == 0) out_tokens[(size_t)b * (K + 1) + d.pos] = y;
}

bool aligned_to(const void* p, size_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

}  // namespace

extern "C" size_t spec_verify_hidden_workspace_bytes(int B, int K, int V) {
    if (B < 1 || B > SV_MAX_BATCH || K < 0 || K > SV_MAX_K || V < 1 || V > SV_MAX_VOCAB) {
        return 0;
    }
    return layout_for(B, K, V).total;
}

extern "C" int spec_verify_hidden(const void* target_hidden, const void* draft_hidden,
                                  const void* head, const int32_t* draft_tokens,
                                  const int32_t* budgets, int B, int K, int H, int V,
                                  float temperature, uint64_t seed, int32_t* out_tokens,
                                  int32_t* out_num_accepted, float* out_p_draft,
                                  float* out_q_draft, int32_t* out_status, void* workspace,
                                  size_t workspace_bytes, void* stream) {
    if (B < 0 || B > SV_MAX_BATCH || K < 0 || K > SV_MAX_K || H < 8 || (H % 8) != 0 ||
        V < 1 || V > SV_MAX_VOCAB || !std::isfinite(temperature) || temperature < 0.0f) {
        return SV_ERR_ARG;
    }
    if (B == 0) return SV_OK;
    const bool greedy = temperature == 0.0f;
    if (!target_hidden || !head || !budgets || !out_tokens || !out_num_accepted || !workspace ||
        (K > 0 && !draft_tokens) || (!greedy && K > 0 && !draft_hidden)) {
        return SV_ERR_NULL;
    }
    if (!aligned_to(target_hidden, 16) || (draft_hidden && !aligned_to(draft_hidden, 16)) ||
        !aligned_to(head, 16) || (draft_tokens && !aligned_to(draft_tokens, 4)) ||
        !aligned_to(budgets, 4) || !aligned_to(out_tokens, 4) ||
        !aligned_to(out_num_accepted, 4) || (out_p_draft && !aligned_to(out_p_draft, 4)) ||
        (out_q_draft && !aligned_to(out_q_draft, 4)) ||
        (out_status && !aligned_to(out_status, 4)) || !aligned_to(workspace, 256)) {
        return SV_ERR_ALIGN;
    }
    const Layout L = layout_for(B, K, V);
    if (workspace_bytes < L.total) return SV_ERR_ARG;

    char* ws = static_cast<char*>(workspace);
    auto i32 = [&](size_t o) { return reinterpret_cast<int32_t*>(ws + o); };
    auto f32 = [&](size_t o) { return reinterpret_cast<float*>(ws + o); };
    const hipStream_t s = static_cast<hipStream_t>(stream);
    const uint16_t* th = static_cast<const uint16_t*>(target_hidden);
    const uint16_t* dh = static_cast<const uint16_t*>(draft_hidden);
    const uint16_t* w = static_cast<const uint16_t*>(head);
    const int rmax = greedy ? B * (K + 1) : (int)packed_rows_max(B, K);
    const double c64 = greedy ? 0.0 : 1.4426950408889634073599246810019 / (double)temperature;

    hipLaunchKernelGGL(hv_plan_kernel, dim3(1), dim3(kPlanThreads), 0, s, budgets, draft_tokens,
                       B, K, V, greedy ? 1 : 0, i32(L.rowmap), i32(L.rowtok), i32(L.off), i32(L.offd),
                       i32(L.nrows), out_status);
    if (hipGetLastError() != hipSuccess) return SV_ERR_HIP;

    const HeadRows rows{th, dh, i32(L.rowmap), B * (K + 1), dh ? B * K : 0, true};
    int rc = svhead::head_stats_launch(rows, w, rmax, i32(L.nrows), H, V, i32(L.rowtok),
                                       temperature, f32(L.sm), greedy ? nullptr : f32(L.ss),
                                       greedy ? nullptr : f32(L.sz), greedy ? i32(L.sa) : nullptr,
                                       ws + L.part, s);
    if (rc != SV_OK) return rc;

    // The draw's path: block masses from the paired product when its
    // many-row form takes the paired rows and the pick kernel's LDS holds the
    // masses and two hidden rows; otherwise the draw rows' logits.
    const HeadRows pair_probe{th, dh, nullptr, B * (K + 1), dh ? B * K : 0, true};
    const bool paired = !greedy && svhead::mass_path(pair_probe, (int)paired_rows_for(B), H, V) &&
                        pick_smem_bytes(V, H) <= kPickSmemMax;
    const int dthreads = 256;
    hipLaunchKernelGGL(hv_decide_kernel, dim3((unsigned)((B + dthreads - 1) / dthreads)),
                       dim3(dthreads), 0, s, budgets, draft_tokens, B, K, V, greedy ? 1 : 0, c64,
                       (uint32_t)(seed & 0xFFFFFFFFull), (uint32_t)(seed >> 32), i32(L.off), i32(L.offd),
                       f32(L.sm), f32(L.ss), f32(L.sz), i32(L.sa), out_tokens, out_num_accepted,
                       out_p_draft, out_q_draft, i32(L.drawmap),
                       reinterpret_cast<DrawDesc*>(ws + L.desc), paired ? 1 : 0);
    if (hipGetLastError() != hipSuccess) return SV_ERR_HIP;
    if (greedy) return SV_OK;

    const HeadRows draw_rows{th, dh, i32(L.drawmap), B * (K + 1), dh ? B * K : 0, true};
    if (paired) {
        // The draw rows' masses from the product's epilogue (no logits
        // written), then one workgroup per request picks the token.
        double* mres = reinterpret_cast<double*>(ws + L.logits);
        double* mpv = mres + 2 * (size_t)B * mass_blocks(V);
        rc = svhead::head_mass_launch(draw_rows, w, (int)paired_rows_for(B), H, V, (float)c64,
                                      DrawMass{reinterpret_cast<const DrawDesc*>(ws + L.desc), mres,
                                               mpv, B},
                                      s);
        if (rc != SV_OK) return rc;
        hipLaunchKernelGGL(hv_pick_kernel, dim3((unsigned)B), dim3(kPickThreads),
                           pick_smem_bytes(V, H), s, th, dh, w, i32(L.drawmap), B * (K + 1), K,
                           H, V, (float)c64, reinterpret_cast<const DrawDesc*>(ws + L.desc), mres,
                           mpv, out_tokens);
        return hipGetLastError() == hipSuccess ? SV_OK : SV_ERR_HIP;
    }
    rc = svhead::head_logits_launch(draw_rows, w, (int)draw_rows_for(B), H, V, f32(L.logits), s);
    if (rc != SV_OK) return rc;
    // 16-byte loads of the fp32 rows when every row starts 16-byte aligned.
    const size_t draw_smem = (size_t)((V + kHvBlock - 1) / kHvBlock) * sizeof(double);
    if (V % 4 == 0) {
        hipLaunchKernelGGL(hv_draw_kernel<true>, dim3((unsigned)B), dim3(kHvDrawThreads), draw_smem,
                           s, f32(L.logits), K, V, (float)c64,
                           reinterpret_cast<const DrawDesc*>(ws + L.desc), out_tokens);
    } else {
        hipLaunchKernelGGL(hv_draw_kernel<false>, dim3((unsigned)B), dim3(kHvDrawThreads), draw_smem,
                           s, f32(L.logits), K, V, (float)c64,
                           reinterpret_cast<const DrawDesc*>(ws + L.desc), out_tokens);
    }
    return hipGetLastError() == hipSuccess ? SV_OK : SV_ERR_HIP;
}
