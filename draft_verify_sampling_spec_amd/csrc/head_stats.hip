// head_stats.hip -- the shared output head with a softmax-statistics
// epilogue, for MI355X (gfx950, MFMA).
//
// What is computed: "Speculative decoding becomes standard: DSpark and
// multi-token drafters", section "What DSpark adds", paragraph 1 (the drafter
// reuses the target's output projection unchanged, so both models' logits for
// a position are that head applied to a hidden state), and section "Why
// draft-and-verify does not change the output", paragraphs 1 and 2 (what a
// verify step needs from each scored row: the target's most likely token, or
// p(x) and q(x) of the drafted token). For hidden states h [R, H] and the head
// W [V, H] (bf16), per row r of z = h W^T: the maximum m, the sum
// S = sum_v 2^((z_v - m) c) with c = log2(e) / T, z at a given token, and the
// first argmax -- without writing z anywhere. The same product can instead
// write the fp32 logits of a few rows (the rows a verify step samples from).
//
// Design: a bf16 matrix product on the matrix cores
// (v_mfma_f32_32x32x16_bf16, fp32 accumulation). A workgroup of 4 waves owns
// a 128-row tile of h and a contiguous range of 128-column tiles of the
// vocabulary (one "split"); per k-step of 64 it stages both operand tiles in
// LDS (the next step's global loads go to registers before the current
// step's products and to LDS after them), and each wave multiplies a
// 64 x 64 quarter as 2 x 2 blocks of 32 x 32. After each vocabulary tile every lane folds its
// accumulators into running per-row statistics of the 32 rows it holds
// (lane l holds column l % 32 of rows 8(i/4) + 4(l/32) + i%4 of a block), so
// no cross-lane work happens per tile; lanes and waves merge once at the end
// and write one partial per (row, split). A second small kernel merges the
// splits. The rows may be gathered through a row map from two buffers, and
// their count may be read on the device (the grid then covers the items of
// any count up to a bound, and workgroups without an item exit).

#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdint>

#include "head_gemm.h"
#include "lds_dma.h"
#include "spec_verify.h"

namespace {

using svhead::DrawDesc;
using svhead::DrawMass;
using svhead::HeadRows;
using svhead::kNoDraw;
using svhead::kResidual;

constexpr int kHThreads = 256;             // 4 waves
constexpr int kTM = 128;                   // rows of h per tile
constexpr int kTN = 128;                   // vocabulary columns per tile
constexpr int kTK = 64;                    // k per staged step
constexpr int kPad = 8;                    // LDS row padding (bf16 elements)
constexpr int kLdsRow = kTK + kPad;        // 72 bf16 = 144 bytes per staged row

constexpr int kResidentSlots = 512;        // one resident wave of workgroups: 2 per CU
constexpr int kAddDeep = 4;                // add-and-store: the two-deep path's k-steps (depth <= 256)

enum Epi { kEpiGreedy = 0, kEpiSampled = 1, kEpiLogits = 2, kEpiAddBf16 = 3 };

// Add-and-store epilogue: row r's output row is out + r * stride (bf16), and
// the value stored there is bf16(base[same place] + logit), one rounding to
// nearest even.
struct RowAdd {
    const uint16_t* base;
    uint16_t* out;
    long long stride;
    svhead::ArgPart* arg;                  // [splits][R] first argmaxes, or NULL
};

constexpr int kTS = kTN + 8;               // staged output tile row (bf16 elements, 272 bytes)

__device__ __forceinline__ uint32_t bf16_rne_bits(float x) {
    const uint32_t u = __float_as_uint(x);
    if ((u & 0x7F800000u) == 0x7F800000u && (u & 0x007FFFFFu) != 0u) return (u >> 16) | 0x0040u;
    return (u + 0x7FFFu + ((u >> 16) & 1u)) >> 16;
}

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

struct HeadPart {                          // one row's statistics over one split
    float m, s, zx;
    int arg;                               // first argmax, INT_MAX if none
};

// Merge (m2, s2) into (m1, s1): both sums are relative to their own maximum.
__device__ __forceinline__ void merge_ms(float& m1, float& s1, float m2, float s2, float c,
                                         bool sampled) {
    const float m = fmaxf(m1, m2);
    if (sampled && m != -INFINITY) {
        const float a = m1 == -INFINITY ? 0.0f : s1 * __builtin_amdgcn_exp2f((m1 - m) * c);
        const float b = m2 == -INFINITY ? 0.0f : s2 * __builtin_amdgcn_exp2f((m2 - m) * c);
        s1 = a + b;
    }
    m1 = m;
}

__device__ __forceinline__ void merge_arg(float& v1, int& i1, float v2, int i2) {
    if (v2 > v1 || (v2 == v1 && i2 < i1)) {
        v1 = v2;
        i1 = i2;
    }
}

// Vocabulary splits: as many as fit one resident wave of workgroups (two per
// CU on 256 CUs) over the row tiles -- a second, partial wave would cost a
// whole workgroup's time -- each split at least eight vocabulary tiles long.
__host__ __device__ inline int splits_for(int R, int V) {
    const int rt = (R + kTM - 1) / kTM, nt = (V + kTN - 1) / kTN;
    int s = kResidentSlots / (rt < 1 ? 1 : rt);
    s = s < 1 ? 1 : s;
    const int cap = (nt + 7) / 8;
    return s > cap ? cap : s;
}

__device__ __forceinline__ int rows_now(int r_max, const int* d_rows) {
    if (!d_rows) return r_max;
    const int r = *d_rows;
    return r < 0 ? 0 : (r > r_max ? r_max : r);
}

// Hidden state of packed row r (NULL: a row of zeros).
__device__ __forceinline__ const uint16_t* row_ptr(const HeadRows& hr, int r, int H) {
    const int v = hr.map ? hr.map[r] : r;
    if (v < 0) return nullptr;
    return v < hr.a_rows ? hr.a + (size_t)v * H : hr.b + (size_t)(v - hr.a_rows) * H;
}

// kEpi: running (max, exp-sum) per row (sampled), (max, first argmax)
// (greedy), or the fp32 logits written to `out` (logits).
template <int kEpi>
__global__ __launch_bounds__(kHThreads) __attribute__((amdgpu_waves_per_eu(2)))
void head_stats_kernel(HeadRows hr, const uint16_t* __restrict__ w, int r_max,
                       const int* __restrict__ d_rows, int H, int V,
                       const int32_t* __restrict__ tok, float c, HeadPart* __restrict__ part,
                       float* __restrict__ out, RowAdd ra) {
    constexpr bool sampled = kEpi == kEpiSampled;
    constexpr bool logits = kEpi == kEpiLogits;
    constexpr bool addbf = kEpi == kEpiAddBf16;
    __shared__ __align__(16) uint16_t As[kTM][kLdsRow];
    __shared__ __align__(16) uint16_t Bs[kTN][kLdsRow];
    __shared__ int tok_s[kTM];             // statistics: the token; logits: row present
    __shared__ float zx_s[kTM];            // the token's logit (one lane of the split finds it)
    __shared__ HeadPart xw[kTM];           // wave-pair merge

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int R = rows_now(r_max, d_rows);
    const int rtiles = (R + kTM - 1) / kTM;
    const int nsplit = splits_for(R, V);
    const int ntiles = (V + kTN - 1) / kTN;
    const int tiles_per_split = (ntiles + nsplit - 1) / nsplit;
    const int wr = (wave >> 1) * 64, wc = (wave & 1) * 64;   // this wave's quarter
    const int nk = (H + kTK - 1) / kTK;

    // One (row tile, split) item per workgroup; workgroups beyond this
    // call's items (a count read on the device) have nothing to do.
    int item = blockIdx.x;
    if (item >= rtiles * nsplit) return;
    if constexpr (addbf || logits) {
        // Workgroups go to the eight XCDs round-robin. Renumber so that a
        // split's row tiles are consecutive workgroups of one XCD: they read
        // the same weight rows at about the same time through one L2. A
        // bijection on [0, rtiles * nsplit) when nsplit is a multiple of 8.
        if (nsplit % 8 == 0) {
            const int xcd = item % 8, slot = item / 8;
            item = ((slot / rtiles) * 8 + xcd) * rtiles + slot % rtiles;
        }
    }
    const int r0 = (item % rtiles) * kTM;
    const int split = item / rtiles;
    const int t0 = split * tiles_per_split, t1 = min(ntiles, t0 + tiles_per_split);

    if (tid < kTM) {
        const bool have = r0 + tid < R;
        if (logits) tok_s[tid] = have && row_ptr(hr, r0 + tid, H) != nullptr;
        else if (addbf) tok_s[tid] = have;
        else tok_s[tid] = (have && tok) ? tok[r0 + tid] : -1;
        zx_s[tid] = NAN;
    }

    // Running statistics of this lane's 32 rows (slot = 16 * br + i): the
    // maximum, and the exp-sum under it (sampled) or the first argmax.
    float rm[32];
    float rx[32];                          // sampled: exp-sum; greedy: argmax bits
    #pragma unroll
    for (int q = 0; q < 32; ++q) {
        rm[q] = -INFINITY;
        rx[q] = sampled ? 0.0f : __int_as_float(INT_MAX);
    }

    // Staging: thread t moves 32 bf16 of row t / 2, k half (t % 2) * 32, of
    // each operand tile per step, as two 16-element pieces.
    const int srow = tid >> 1, skh = (tid & 1) * 32;
    const uint16_t* arow = r0 + srow < R ? row_ptr(hr, r0 + srow, H) : nullptr;
    auto load16 = [&](const uint16_t* rowp, int k, uint4& x0, uint4& x1) {
        x0 = make_uint4(0u, 0u, 0u, 0u);
        x1 = x0;
        if (rowp) {
            const uint16_t* p = rowp + k;
            if (k + 16 <= H) {
                x0 = *reinterpret_cast<const uint4*>(p);
                x1 = *reinterpret_cast<const uint4*>(p + 8);
            } else {
                // The row's last step: elements at or beyond H read as 0.
                uint32_t wd[8];
                #pragma unroll
                for (int j = 0; j < 8; ++j) {
                    const uint32_t lo = k + 2 * j < H ? p[2 * j] : 0u;
                    const uint32_t hi = k + 2 * j + 1 < H ? p[2 * j + 1] : 0u;
                    wd[j] = lo | (hi << 16);
                }
                x0 = make_uint4(wd[0], wd[1], wd[2], wd[3]);
                x1 = make_uint4(wd[4], wd[5], wd[6], wd[7]);
            }
        }
    };
    struct Piece {
        uint4 a0, a1, a2, a3, b0, b1, b2, b3;
    };
    // Depth a multiple of kTK: every load is a full 16-byte load from a valid
    // row (a missing row reads the weight's first row), and missing rows
    // are zeroed by masks as the words are staged. Not in the greedy
    // statistics, whose registers it would push into spills.
    const bool hfull = kEpi != kEpiGreedy && H % kTK == 0;
    const uint32_t mask_a = arow ? 0xFFFFFFFFu : 0u;
    uint32_t mask_b = 0xFFFFFFFFu;
    auto load_step = [&](int v0, int k0, Piece& pc) {
        const uint16_t* brow = v0 + srow < V ? w + (size_t)(v0 + srow) * H : nullptr;
        if (hfull) {
            const uint16_t* pa = (arow ? arow : w) + k0 + skh;
            const uint16_t* pb = (brow ? brow : w) + k0 + skh;
            pc.a0 = *reinterpret_cast<const uint4*>(pa);
            pc.a1 = *reinterpret_cast<const uint4*>(pa + 8);
            pc.a2 = *reinterpret_cast<const uint4*>(pa + 16);
            pc.a3 = *reinterpret_cast<const uint4*>(pa + 24);
            pc.b0 = *reinterpret_cast<const uint4*>(pb);
            pc.b1 = *reinterpret_cast<const uint4*>(pb + 8);
            pc.b2 = *reinterpret_cast<const uint4*>(pb + 16);
            pc.b3 = *reinterpret_cast<const uint4*>(pb + 24);
            mask_b = brow ? 0xFFFFFFFFu : 0u;
            return;
        }
        load16(arow, k0 + skh, pc.a0, pc.a1);
        load16(arow, k0 + skh + 16, pc.a2, pc.a3);
        load16(brow, k0 + skh, pc.b0, pc.b1);
        load16(brow, k0 + skh + 16, pc.b2, pc.b3);
    };
    auto store_step = [&](const Piece& pc) {
        uint4* ra = reinterpret_cast<uint4*>(&As[srow][skh]);
        uint4* rb = reinterpret_cast<uint4*>(&Bs[srow][skh]);
        const uint32_t ma = hfull ? mask_a : 0xFFFFFFFFu, mb = hfull ? mask_b : 0xFFFFFFFFu;
        auto m = [](const uint4& x, uint32_t k) { return make_uint4(x.x & k, x.y & k, x.z & k, x.w & k); };
        ra[0] = m(pc.a0, ma); ra[1] = m(pc.a1, ma); ra[2] = m(pc.a2, ma); ra[3] = m(pc.a3, ma);
        rb[0] = m(pc.b0, mb); rb[1] = m(pc.b1, mb); rb[2] = m(pc.b2, mb); rb[3] = m(pc.b3, mb);
    };

    // Add-and-store: this thread's running first argmax over the values it
    // stores (its row, its half of every tile's columns, in column order).
    float am_v = -INFINITY;
    int am_i = INT_MAX;

    for (int t = t0; t < t1; ++t) {
        const int v0 = t * kTN;
        Piece bp;                          // add-and-store: this thread's 8 backbone groups,
        bool pre = false;                  // loaded during the product
        f32x16 acc[2][2];
        #pragma unroll
        for (int a = 0; a < 2; ++a)
            #pragma unroll
            for (int b = 0; b < 2; ++b)
                #pragma unroll
                for (int i = 0; i < 16; ++i) acc[a][b][i] = 0.0f;

        if constexpr (addbf) {
            if (nk <= kAddDeep && H % kTK == 0) {
                // A shallow product (the Markov head's rank): two k-steps'
                // operand loads in flight instead of one. Every step is full
                // depth, so the loads take no ragged-tail path: a missing row
                // reads the weight's first row and is zeroed afterwards, and
                // every lane issues the same loads, which lets each step wait
                // for its own loads only.
                const uint16_t* brow = v0 + srow < V ? w + (size_t)(v0 + srow) * H : nullptr;
                const uint16_t* pa = (arow ? arow : w) + skh;
                const uint16_t* pb = (brow ? brow : w) + skh;
                // Missing rows are zeroed by masking the words as they are
                // staged (a select at the load would split it into 4-byte
                // loads, and masking there would wait for it at once).
                const uint32_t ma = arow ? 0xFFFFFFFFu : 0u, mb = brow ? 0xFFFFFFFFu : 0u;
                auto ld = [&](const uint16_t* p, int k) -> uint4 {
                    return *reinterpret_cast<const uint4*>(p + k);
                };
                auto fetch = [&](int k0) -> Piece {
                    Piece pc;
                    pc.a0 = ld(pa, k0);
                    pc.a1 = ld(pa, k0 + 8);
                    pc.a2 = ld(pa, k0 + 16);
                    pc.a3 = ld(pa, k0 + 24);
                    pc.b0 = ld(pb, k0);
                    pc.b1 = ld(pb, k0 + 8);
                    pc.b2 = ld(pb, k0 + 16);
                    pc.b3 = ld(pb, k0 + 24);
                    return pc;
                };
                auto mk = [](const uint4& x, uint32_t m) {
                    return make_uint4(x.x & m, x.y & m, x.z & m, x.w & m);
                };
                auto stage = [&](const Piece& pc) {
                    uint4* sa = reinterpret_cast<uint4*>(&As[srow][skh]);
                    uint4* sb = reinterpret_cast<uint4*>(&Bs[srow][skh]);
                    sa[0] = mk(pc.a0, ma); sa[1] = mk(pc.a1, ma); sa[2] = mk(pc.a2, ma); sa[3] = mk(pc.a3, ma);
                    sb[0] = mk(pc.b0, mb); sb[1] = mk(pc.b1, mb); sb[2] = mk(pc.b2, mb); sb[3] = mk(pc.b3, mb);
                };
                auto mma = [&]() {
                    #pragma unroll
                    for (int kk = 0; kk < kTK; kk += 16) {
                        bf16x8 af[2], bfr[2];
                        #pragma unroll
                        for (int a = 0; a < 2; ++a) {
                            af[a] = *reinterpret_cast<const bf16x8*>(
                                &As[wr + 32 * a + (lane & 31)][kk + (lane >> 5) * 8]);
                            bfr[a] = *reinterpret_cast<const bf16x8*>(
                                &Bs[wc + 32 * a + (lane & 31)][kk + (lane >> 5) * 8]);
                        }
                        #pragma unroll
                        for (int a = 0; a < 2; ++a)
                            #pragma unroll
                            for (int b = 0; b < 2; ++b)
                                acc[a][b] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[a], bfr[b], acc[a][b], 0, 0, 0);
                    }
                };
                // Steps 0 and 1 go out together; step ks + 2 as soon as step
                // ks is staged. Every fetch is unconditional, so no wait
                // hides behind a branch; a step past the last is the last
                // step again (in bounds, not used).
                auto kstep = [&](int st) { return (st < nk ? st : nk - 1) * kTK; };
                Piece p0 = fetch(0);
                Piece p1 = fetch(kstep(1));
                __syncthreads();           // earlier readers of the operand tiles are done
                stage(p0);
                p0 = fetch(kstep(2));
                if ((V & 7) == 0) {
                    // The tile's backbone groups (epilogue step 1) go out now,
                    // behind the operand loads. Absent rows read the tile's
                    // first row and columns past V the row's last group
                    // (in bounds; neither is stored).
                    const int rr = min(r0 + (tid >> 1), R - 1);
                    const uint16_t* src = ra.base + (size_t)rr * (size_t)ra.stride;
                    const int c0 = v0 + (tid & 1) * 64;
                    auto grp = [&](int q8) {
                        return *reinterpret_cast<const uint4*>(src + min(c0 + q8 * 8, V - 8));
                    };
                    bp.a0 = grp(0); bp.a1 = grp(1); bp.a2 = grp(2); bp.a3 = grp(3);
                    bp.b0 = grp(4); bp.b1 = grp(5); bp.b2 = grp(6); bp.b3 = grp(7);
                    pre = true;
                }
                __syncthreads();
                mma();
                if (nk > 1) {
                    __syncthreads();
                    stage(p1);
                    p1 = fetch(kstep(3));
                    __syncthreads();
                    mma();
                }
                if (nk > 2) {
                    __syncthreads();
                    stage(p0);
                    __syncthreads();
                    mma();
                }
                if (nk > 3) {
                    __syncthreads();
                    stage(p1);
                    __syncthreads();
                    mma();
                }
                goto epilogue;
            }
        }
        {
        Piece pc;
        load_step(v0, 0, pc);
        __syncthreads();                   // previous tile's readers are done
        store_step(pc);
        __syncthreads();
        for (int ks = 0; ks < nk; ++ks) {
            const bool more = ks + 1 < nk;
            if (more) load_step(v0, (ks + 1) * kTK, pc);
            #pragma unroll
            for (int kk = 0; kk < kTK; kk += 16) {
                bf16x8 af[2], bfr[2];
                #pragma unroll
                for (int a = 0; a < 2; ++a) {
                    af[a] = *reinterpret_cast<const bf16x8*>(
                        &As[wr + 32 * a + (lane & 31)][kk + (lane >> 5) * 8]);
                    bfr[a] = *reinterpret_cast<const bf16x8*>(
                        &Bs[wc + 32 * a + (lane & 31)][kk + (lane >> 5) * 8]);
                }
                #pragma unroll
                for (int a = 0; a < 2; ++a)
                    #pragma unroll
                    for (int b = 0; b < 2; ++b)
                        acc[a][b] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[a], bfr[b], acc[a][b], 0, 0, 0);
            }
            __syncthreads();
            if (more) {
                store_step(pc);
                __syncthreads();
            }
        }
        }
    epilogue:

        if (logits) {
            // The tile's logits, one row segment of 32 columns per block.
            #pragma unroll
            for (int a = 0; a < 2; ++a) {
                #pragma unroll
                for (int i = 0; i < 16; ++i) {
                    const int rl = wr + 32 * a + 8 * (i >> 2) + 4 * (lane >> 5) + (i & 3);
                    if (!tok_s[rl]) continue;
                    #pragma unroll
                    for (int b = 0; b < 2; ++b) {
                        const int col = v0 + wc + 32 * b + (lane & 31);
                        if (col < V) out[(size_t)(r0 + rl) * V + col] = acc[a][b][i];
                    }
                }
            }
            continue;
        }
        if constexpr (addbf) {
            // The staged output tile (this instantiation only). The previous
            // tile's stores from it ended before the barrier that opened
            // this tile's product.
            __shared__ __align__(16) uint16_t T[kTM * kTS];
            // 1. The tile's backbone values into LDS, 16-byte loads: thread
            //    t takes row t / 2, columns (t % 2) * 64 .. + 64.
            const int trow = tid >> 1, tc0 = (tid & 1) * 64;
            const bool rok = tok_s[trow] != 0;
            const size_t goff = (size_t)(r0 + trow) * (size_t)ra.stride + (size_t)(v0 + tc0);
            const bool vec = (V & 7) == 0;         // 16-byte aligned rows and columns
            if (pre) {
                uint4* dst = reinterpret_cast<uint4*>(&T[trow * kTS + tc0]);
                dst[0] = bp.a0; dst[1] = bp.a1; dst[2] = bp.a2; dst[3] = bp.a3;
                dst[4] = bp.b0; dst[5] = bp.b1; dst[6] = bp.b2; dst[7] = bp.b3;
            } else if (rok) {
                #pragma unroll
                for (int q8 = 0; q8 < 8; ++q8) {
                    const int col = v0 + tc0 + q8 * 8;
                    uint4 x = make_uint4(0u, 0u, 0u, 0u);
                    if (vec && col + 8 <= V) {
                        x = *reinterpret_cast<const uint4*>(ra.base + goff + q8 * 8);
                    } else if (col < V) {
                        uint32_t wd[4] = {0u, 0u, 0u, 0u};
                        for (int e = 0; e < 8 && col + e < V; ++e)
                            wd[e >> 1] |= (uint32_t)ra.base[goff + q8 * 8 + e] << ((e & 1) * 16);
                        x = make_uint4(wd[0], wd[1], wd[2], wd[3]);
                    }
                    *reinterpret_cast<uint4*>(&T[trow * kTS + tc0 + q8 * 8]) = x;
                }
            }
            __syncthreads();
            // 2. Each lane adds its accumulators in place, one rounding.
            #pragma unroll
            for (int a = 0; a < 2; ++a) {
                #pragma unroll
                for (int i = 0; i < 16; ++i) {
                    const int rl = wr + 32 * a + 8 * (i >> 2) + 4 * (lane >> 5) + (i & 3);
                    #pragma unroll
                    for (int b = 0; b < 2; ++b) {
                        const int cl = wc + 32 * b + (lane & 31);
                        uint16_t& cell = T[rl * kTS + cl];
                        const float sum = __uint_as_float((uint32_t)cell << 16) + acc[a][b][i];
                        cell = (uint16_t)bf16_rne_bits(sum);
                    }
                }
            }
            __syncthreads();
            // 3. The tile back out, 16-byte stores; the first argmax follows
            //    the stored values in column order (a strictly larger value
            //    replaces it, so the lowest column wins ties).
            if (rok) {
                #pragma unroll
                for (int q8 = 0; q8 < 8; ++q8) {
                    const int col = v0 + tc0 + q8 * 8;
                    const uint4 x = *reinterpret_cast<const uint4*>(&T[trow * kTS + tc0 + q8 * 8]);
                    const uint32_t wd[4] = {x.x, x.y, x.z, x.w};
                    if (vec && col + 8 <= V) {
                        *reinterpret_cast<uint4*>(ra.out + goff + q8 * 8) = x;
                    } else if (col < V) {
                        for (int e = 0; e < 8 && col + e < V; ++e)
                            ra.out[goff + q8 * 8 + e] = (uint16_t)(wd[e >> 1] >> ((e & 1) * 16));
                    }
                    if (ra.arg) {
                        float f[8];
                        #pragma unroll
                        for (int e = 0; e < 8; ++e)
                            f[e] = __uint_as_float((wd[e >> 1] >> ((e & 1) * 16)) << 16);
                        if (col + 8 <= V) {
                            // The group's maximum first (NaN never wins); only
                            // a group that beats the running value is searched
                            // for its first column holding that maximum.
                            const float g = fmaxf(fmaxf(fmaxf(f[0], f[1]), fmaxf(f[2], f[3])),
                                                  fmaxf(fmaxf(f[4], f[5]), fmaxf(f[6], f[7])));
                            if (g > am_v) {
                                int e0 = 7;
                                #pragma unroll
                                for (int e = 6; e >= 0; --e) e0 = f[e] == g ? e : e0;
                                am_v = g;
                                am_i = col + e0;
                            }
                        } else {
                            #pragma unroll
                            for (int e = 0; e < 8; ++e) {
                                if (col + e < V && f[e] > am_v) {
                                    am_v = f[e];
                                    am_i = col + e;
                                }
                            }
                        }
                    }
                }
            }
            continue;
        }
        // Fold the tile into the lane's running row statistics, without
        // branches: columns past V (the last tile only) read as -inf; the
        // sampled sum is rescaled once per row slot and tile.
        const bool full = v0 + kTN <= V;
        const int col0 = v0 + wc + (lane & 31), col1 = col0 + 32;
        #pragma unroll
        for (int a = 0; a < 2; ++a) {
            #pragma unroll
            for (int i = 0; i < 16; ++i) {
                const int q = 16 * a + i;
                float z0 = acc[a][0][i], z1 = acc[a][1][i];
                if (!full) {
                    z0 = col0 < V ? z0 : -INFINITY;
                    z1 = col1 < V ? z1 : -INFINITY;
                }
                if (sampled) {
                    const float mn = fmaxf(rm[q], fmaxf(z0, z1));
                    const float mr = mn == -INFINITY ? 0.0f : mn;   // all -inf so far: terms stay 0
                    rx[q] = rx[q] * __builtin_amdgcn_exp2f((rm[q] - mr) * c) +
                            __builtin_amdgcn_exp2f((z0 - mr) * c) +
                            __builtin_amdgcn_exp2f((z1 - mr) * c);
                    rm[q] = mn;
                } else {
                    // A lane's columns go up, so the first maximum wins.
                    const bool b0 = z0 > rm[q];
                    rm[q] = b0 ? z0 : rm[q];
                    rx[q] = b0 ? __int_as_float(col0) : rx[q];
                    const bool b1 = z1 > rm[q];
                    rm[q] = b1 ? z1 : rm[q];
                    rx[q] = b1 ? __int_as_float(col1) : rx[q];
                }
                // The drafted token's logit: one lane of the row's split.
                const int rl = wr + 32 * a + 8 * (i >> 2) + 4 * (lane >> 5) + (i & 3);
                const int x = tok_s[rl];
                if (x == col0 || x == col1) zx_s[rl] = x == col0 ? z0 : z1;
            }
        }
    }

    if constexpr (addbf) {
        if (ra.arg) {
            // A row's two threads (lanes 2m and 2m + 1, the tiles' two column
            // halves) merge; the first writes the split's entry.
            merge_arg(am_v, am_i, __shfl_xor(am_v, 1, 64), __shfl_xor(am_i, 1, 64));
            const int trow = tid >> 1;
            if ((tid & 1) == 0 && r0 + trow < R)
                ra.arg[(size_t)split * R + r0 + trow] = svhead::ArgPart{am_v, am_i};
        }
    }
    if (logits || addbf) return;
    // Lanes holding the same rows (same l / 32 half): merge across columns.
    #pragma unroll
    for (int q = 0; q < 32; ++q) {
        float m = rm[q], x = rx[q];
        #pragma unroll
        for (int o = 1; o < 32; o <<= 1) {
            const float m2 = __shfl_xor(m, o, 64), x2 = __shfl_xor(x, o, 64);
            if (sampled) {
                merge_ms(m, x, m2, x2, c, true);
            } else {
                int ai = __float_as_int(x);
                merge_arg(m, ai, m2, __float_as_int(x2));
                x = __int_as_float(ai);
            }
        }
        rm[q] = m;
        rx[q] = x;
    }
    // Waves with the same rows (wave and wave ^ 1) merge through LDS.
    __syncthreads();
    if ((wave & 1) == 1 && (lane & 31) == 0) {
        #pragma unroll
        for (int q = 0; q < 32; ++q) {
            const int a = q >> 4, i = q & 15;
            const int rl = wr + 32 * a + 8 * (i >> 2) + 4 * (lane >> 5) + (i & 3);
            xw[rl] = HeadPart{rm[q], sampled ? rx[q] : 0.0f, 0.0f,
                              sampled ? INT_MAX : __float_as_int(rx[q])};
        }
    }
    __syncthreads();
    if ((wave & 1) == 0 && (lane & 31) == 0) {
        #pragma unroll
        for (int q = 0; q < 32; ++q) {
            const int a = q >> 4, i = q & 15;
            const int rl = wr + 32 * a + 8 * (i >> 2) + 4 * (lane >> 5) + (i & 3);
            const HeadPart o = xw[rl];
            HeadPart out;
            out.m = rm[q];
            out.zx = zx_s[rl];
            if (sampled) {
                out.s = rx[q];
                merge_ms(out.m, out.s, o.m, o.s, c, true);
                out.arg = INT_MAX;
            } else {
                out.s = 0.0f;
                out.arg = __float_as_int(rx[q]);
                merge_arg(out.m, out.arg, o.m, o.arg);
            }
            if (r0 + rl < R) part[(size_t)split * R + r0 + rl] = out;
        }
    }
}

// ------------------------------------------- the product for many rows --

// For many rows (a verify batch's scored rows) the product above is bound by
// LDS traffic (64 FLOP per staged byte at 128 x 128 tiles) and re-streams
// each workgroup's hidden-state tile from beyond the L2 for every vocabulary
// tile. This kernel instead gives each workgroup a 256 x 256 tile, four
// waves of 128 x 128 (16 blocks of 32 x 32, 256 accumulators per lane), and
// stages k-steps of 64 through two LDS buffers filled by buffer-to-LDS
// 16-byte loads (no registers in between). A k-step of 64 gives each row
// one whole 128-byte line per load: the L2 serves whole lines at about
// twice the rate of half lines, and a CU needs about 32 bytes a clock to
// keep its matrix cores busy on this tile. Each step's 64 of k is
// multiplied as four groups of 16; the workgroup synchronises before a
// step's last group, so the load of the step after next goes out a whole
// step before it is needed. (Buffer loads rather than global ones: with a
// global load to LDS in flight the compiler must assume it may also count
// as an LDS access and drains every LDS read before the first product; with
// buffer loads it waits only for the fragments it uses. Their range check
// also reads rows past the vocabulary and rows of zeros as zeros.) The
// workgroups of one XCD work together on a 6 x 5 super-tile -- six row
// tiles (a "band") by five vocabulary tiles -- and move it along the
// vocabulary, so the operands one step needs are shared through that XCD's
// L2, and each workgroup keeps one row tile while its running row
// statistics stay in registers. One workgroup per CU; the schedule assumes
// the dispatcher deals workgroups to the XCDs round-robin (correct under
// any dealing, only slower).
constexpr int kBM = 256, kBN = 256, kBK = 64;
constexpr int kMmThreads = 256;
constexpr int kBandTiles = 6;                        // row tiles per band (statistics)
constexpr int kColTiles = 5;                         // vocabulary tiles per super-step (statistics)
constexpr int kLogBand = 4, kLogCols = 8;            // the same for logits (few rows)
constexpr int kXcds = 8;
constexpr int kMmParts = kXcds * kColTiles;          // partials per row
constexpr int kMmGrid = kXcds * 32;                  // one workgroup per CU
constexpr int kMmOpBytes = kBM * kBK * 2;            // one operand of one stage (32 KB)
constexpr int kMmLds = 2 * 2 * kMmOpBytes;           // two stages, both operands
constexpr unsigned kMmOob = 0x80000000u;             // a buffer offset past every range below
enum MmMode { kMmGreedy = 0, kMmSampled = 1, kMmLogits = 2, kMmMass = 3 };

// Side workgroups. An XCD's CUs beyond its kB x kC super-tile (two at 6 x 5)
// take the vocabulary's last side_cols tiles, for every row tile, column by
// column; the super-tiles keep the first kC * spb tiles. spb balances the
// two: a super-tile workgroup takes about nb * spb / 8 tiles (nb bands), a
// side one side_cols * rtiles / (8 * side workgroups per XCD) -- about a
// sixteenth of the vocabulary when the bands are whole. spb stays at least
// 8, so that every XCD has a super-step in every band, and side_cols at
// most mm_side_max(V) (the workspace's bound). Both the product and the
// merge of its partials compute it from the row count.
struct MmSplit {
    int spb, side_cols;
};
__host__ __device__ inline int mm_side_max(int V) { return (V + kBN - 1) / kBN / 16 + 4; }
template <int kB, int kC>
__host__ __device__ inline MmSplit mm_split(int R, int V) {
    const int rtiles = (R + kBM - 1) / kBM, ntiles = (V + kBN - 1) / kBN;
    const int nb = (rtiles + kB - 1) / kB;
    const int s_all = (ntiles + kC - 1) / kC;
    constexpr int kSide = 32 - kB * kC;
    MmSplit best{s_all, 0};
    if (kSide <= 0 || R < 1) return best;
    long long best_cost = ((long long)nb * s_all + kXcds - 1) / kXcds;
    for (int sp = s_all - 1; sp >= kXcds; --sp) {
        const int side = ntiles - kC * sp;
        if (side > mm_side_max(V)) break;
        const long long tm = ((long long)nb * sp + kXcds - 1) / kXcds;
        const long long ts = ((long long)side * rtiles + kXcds * kSide - 1) / (kXcds * kSide);
        const long long cost = tm > ts ? tm : ts;
        if (cost < best_cost) {
            best_cost = cost;
            best = MmSplit{sp, side};
        }
    }
    return best;
}

// Row and column counts for which a call takes this path with super-tiles
// of kB row tiles by kC vocabulary tiles (the workspace is sized from these
// alone): at least one full band, and every XCD with a super-step in every
// band.
template <int kB, int kC>
__host__ __device__ inline bool mm_shape_t(int r_max, int V) {
    return r_max >= kBM * kB && (V + kBN - 1) / kBN >= kC * kXcds;
}
__host__ __device__ inline bool mm_shape(int r_max, int V) {
    return mm_shape_t<kBandTiles, kColTiles>(r_max, V);
}

// The whole condition: the shape, whole k-steps, rows of the two buffers in
// separate groups of 8 (one load instruction reads one group through one
// buffer descriptor), and byte offsets within each hidden-state buffer and
// within a vocabulary tile that stay below kMmOob (32-bit buffer offsets).
template <int kB, int kC>
inline bool mm_path(const HeadRows& hr, int r_max, int H, int V) {
    const unsigned long long row = 2ull * (unsigned long long)H;
    return mm_shape_t<kB, kC>(r_max, V) && H % kBK == 0 && row * kBN <= kMmOob / 2 &&
           (hr.b_rows == 0 || hr.grouped8) &&
           row * (unsigned long long)hr.a_rows <= kMmOob &&
           row * (unsigned long long)hr.b_rows <= kMmOob;
}

using svdma::ring_barrier;
using svdma::wait_vm;

__device__ __forceinline__ __amdgpu_buffer_rsrc_t mm_rsrc(const void* p, unsigned n) {
    return svdma::rsrc(p, n);
}
__device__ __forceinline__ void lds_load16(__amdgpu_buffer_rsrc_t r, unsigned off,
                                           unsigned char* lds) {
    svdma::load16(r, off, lds);
}

// kMode: the row statistics (greedy or sampled, partials per (XCD, column
// slot) into part), the fp32 logits themselves (into out, row-major,
// R x V), or the draw masses of paired draw rows (into dm). kBandT x kColT:
// the XCD's super-tile.
template <int kMode, int kBandT, int kColT>
__global__ __launch_bounds__(kMmThreads) __attribute__((amdgpu_waves_per_eu(1, 1)))
void head_mm_kernel(HeadRows hr, const uint16_t* __restrict__ w, int r_max,
                    const int* __restrict__ d_rows, int H, int V,
                    const int32_t* __restrict__ tok, float c, HeadPart* __restrict__ part,
                    float* __restrict__ out, DrawMass dm) {
    constexpr bool kSampled = kMode == kMmSampled;
    constexpr bool kLogits = kMode == kMmLogits;
    constexpr bool kMass = kMode == kMmMass;
    constexpr bool kRowStats = !kLogits && !kMass;
    extern __shared__ __align__(16) unsigned char mm_smem[];
    __shared__ HeadPart xw[kBM];

    // The wave index in a scalar register, so that the loads' LDS
    // destinations (M0) are formed by scalar instructions.
    const int tid = threadIdx.x, lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    // Wave (wm, wn): hidden rows wm * 128 .. + 128 of the row tile and
    // vocabulary columns wn * 128 .. + 128 of the vocabulary tile. The
    // product is formed transposed (head rows as the first operand), so in
    // each 32 x 32 block a lane holds one hidden row (lane % 32) and 16 of
    // the block's vocabulary columns: a lane's statistics cover 4 rows.
    const int wm = wave >> 1, wn = wave & 1;
    const int R = rows_now(r_max, d_rows);
    const int xcd = (int)blockIdx.x % kXcds, slot = (int)blockIdx.x / kXcds;
    constexpr int kSuper = kBandT * kColT, kSide = 32 - kSuper;
    constexpr int kSideN = kSide > 0 ? kSide : 1;     // (divisor; no side workgroups when kSide is 0)
    const MmSplit split = mm_split<kBandT, kColT>(R, V);
    const bool side = slot >= kSuper;                // a side workgroup (see mm_split)
    if (R == 0 || (side && split.side_cols == 0)) return;
    const int rt_in = side ? 0 : slot % kBandT, vt = side ? 0 : slot / kBandT;
    const int rtiles = (R + kBM - 1) / kBM;
    const int nbands = (rtiles + kBandT - 1) / kBandT;
    const int ntiles = (V + kBN - 1) / kBN;
    const int spb = split.spb;                       // super-steps per band
    const int ncm = ntiles - split.side_cols;        // the super-tiles' vocabulary tiles
    // A side workgroup's tiles: t_beg .. t_end - 1 of the side region's
    // side_cols * rtiles tiles, numbered column-major (a column's row tiles
    // in turn, so its head rows stay in the L2).
    const int sw = xcd * kSide + (slot - kSuper);
    const long long n_side = (long long)split.side_cols * rtiles;
    const int t_beg = side ? (int)(sw * n_side / (kXcds * kSideN)) : 0;
    const int total = side ? (int)((sw + 1) * n_side / (kXcds * kSideN)) : nbands * spb;
    const int stride = side ? 1 : kXcds;
    const int nk = H / kBK;

    // The workgroup's tiles, in order. Super-tile workgroups: super-steps
    // stp = xcd, xcd + 8, ...; super-step stp covers row tile
    // (stp / spb) * kBandT + rt_in and vocabulary tile (stp % spb) * kColT +
    // vt, skipped when either lies past the end (every band that has this
    // row tile has at least one vocabulary tile here: spb >= 8, and with
    // side columns every group of kColT is whole). Side workgroups: tile t
    // covers row tile t % rtiles and vocabulary tile ncm + t / rtiles, and
    // each is its own band, written to its column's partial slot.
    auto row0_of = [&](int stp) {
        return (side ? stp % rtiles : stp / spb * kBandT + rt_in) * kBM;
    };
    auto v0_of = [&](int stp) {
        return (side ? ncm + stp / rtiles : (stp % spb) * kColT + vt) * kBN;
    };
    auto band_of = [&](int stp) { return side ? stp : stp / spb; };
    auto pslot_of = [&](int stp) {
        return side ? kXcds * kColT + stp / rtiles : xcd * kColT + vt;
    };
    auto next_tile = [&](int stp) {
        while (stp < total && (row0_of(stp) >= R || v0_of(stp) >= V)) stp += stride;
        return stp < total ? stp : total;
    };

    // ---- loads: the hidden and head rows of one k-step into one of two
    // LDS stages. Instruction j of wave w moves rows 8q .. 8q + 7 of an
    // operand tile (q = 8w + j), one 16-byte piece per lane, 8 lanes a row.
    // Row r's k-piece kc (of 8) sits at piece position kc ^ ((r / 2) % 8) of
    // its 128-byte LDS row, so a fragment read (16 rows at one k-piece per
    // 256-byte bank sweep) touches every bank once; the piece a lane moves
    // depends on the parity of q (rows 8q .. 8q + 7 have (r / 2) % 8 =
    // 4 (q % 2) + lane / 16).
    const int lrow = lane >> 3;
    const int lkc0 = (lane & 7) ^ ((lane >> 4) & 7);         // even q
    const int lkc1 = (lane & 7) ^ ((4 + (lane >> 4)) & 7);   // odd q
    const unsigned hrow_bytes = 2u * (unsigned)H;
    const __amdgpu_buffer_rsrc_t rsrc_a = mm_rsrc(hr.a, hrow_bytes * (unsigned)hr.a_rows);
    const __amdgpu_buffer_rsrc_t rsrc_b = mm_rsrc(hr.b, hrow_bytes * (unsigned)hr.b_rows);
    __amdgpu_buffer_rsrc_t rsrc_w = rsrc_a;          // head rows of the loader's vocabulary tile
    // Hidden rows of the loader's band: this lane's byte offsets (a row of
    // zeros: out of range) and, in bit j (the same in every lane), whether
    // instruction j's rows are rows of b. The rows of one instruction come
    // from one buffer (the path's condition); a row of zeros reads zeros
    // from either.
    unsigned hoff[8];
    unsigned hbu = 0;
    int l_band = -1;
    auto set_rows = [&](int r0) {
        int vr[8];                                   // the row map's entries, loaded together
        #pragma unroll
        for (int j = 0; j < 8; ++j) {
            int r = r0 + 8 * (wave * 8 + j) + lrow;
            r = r < R ? r : R - 1;
            vr[j] = hr.map ? hr.map[r] : r;
        }
        hbu = 0;
        #pragma unroll
        for (int j = 0; j < 8; ++j) {
            const int v = vr[j];
            const bool in_b = v >= hr.a_rows;
            hoff[j] = v < 0 ? kMmOob
                            : (unsigned)(in_b ? v - hr.a_rows : v) * hrow_bytes +
                                  16u * (unsigned)((j & 1) ? lkc1 : lkc0);
            hbu |= __builtin_amdgcn_ballot_w64(in_b) != 0 ? 1u << j : 0u;
        }
    };
    // The loader walks the same steps as the product, ahead of it: l_stp,
    // l_ks is the step whose loads go out next (l_stp == total: none).
    int l_stp = total, l_ks = 0;
    auto loader_at = [&](int stp) {
        l_stp = stp;
        l_ks = 0;
        if (stp >= total) return;
        const int v0 = v0_of(stp);
        // Head rows v0 .. v0 + 255; rows past V read as zeros.
        rsrc_w = mm_rsrc(w + (size_t)v0 * H, (unsigned)min(kBN, V - v0) * hrow_bytes);
        const int band = band_of(stp);
        if (band != l_band) {
            l_band = band;
            set_rows(row0_of(stp));
        }
    };
    // Load i (0 .. 15) of the loader's step into stage st: row group i / 2,
    // head rows when i is odd.
    auto load_one = [&](int st, int i) {
        const int j = i >> 1, q = wave * 8 + j;
        const unsigned k0b = 2u * (unsigned)(l_ks * kBK);
        unsigned char* dst = mm_smem + st * 2 * kMmOpBytes + q * 1024;
        if (i & 1) {
            lds_load16(rsrc_w, (unsigned)(8 * q + lrow) * hrow_bytes +
                                   16u * (unsigned)((j & 1) ? lkc1 : lkc0) + k0b,
                       dst + kMmOpBytes);
        } else {
            lds_load16(((hbu >> j) & 1u) ? rsrc_b : rsrc_a, hoff[j] + k0b, dst);
        }
    };
    auto loader_next = [&]() {
        if (l_stp < total && ++l_ks == nk) loader_at(next_tile(l_stp + stride));
    };

    // ---- the product: 16 blocks of 32 x 32 per wave, fragments of one
    // group (16 of k) at a time.
    f32x16 acc[4][4];                                // [vocabulary block][hidden block]
    struct Frags { bf16x8 h[4], w[4]; };
    auto read_frags = [&](Frags& f, int st, int kk) {
        const unsigned char* sh_h = mm_smem + st * 2 * kMmOpBytes;
        const unsigned char* sh_w = sh_h + kMmOpBytes;
        // Row r's piece 2kk + lane / 32 sits at position piece ^ ((r / 2) % 8);
        // the blocks start at multiples of 32.
        const int piece = ((2 * kk + (lane >> 5)) ^ ((lane >> 1) & 7)) << 4;
        #pragma unroll
        for (int a = 0; a < 4; ++a) {
            f.h[a] = *reinterpret_cast<const bf16x8*>(sh_h + (wm * 128 + 32 * a + (lane & 31)) * 128 + piece);
            f.w[a] = *reinterpret_cast<const bf16x8*>(sh_w + (wn * 128 + 32 * a + (lane & 31)) * 128 + piece);
        }
    };
    auto multiply = [&](const Frags& f) {
        #pragma unroll
        for (int b2 = 0; b2 < 4; ++b2)
            #pragma unroll
            for (int a = 0; a < 4; ++a)
                acc[b2][a] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(f.w[b2], f.h[a], acc[b2][a], 0, 0, 0);
    };
    // The same 16 products with loads i0 .. i0 + 7 of the loader's step
    // placed one after every second product, so the address unit takes them
    // while the matrix cores work instead of stalling the wave. The loads go
    // out even past the end of the stream (they then refill a stage nobody
    // reads again): no branch among the products.
    auto multiply_ld = [&](const Frags& f, int st, int i0) {
        #pragma unroll
        for (int u = 0; u < 16; ++u) {
            const int b2 = u >> 2, a = u & 3;
            acc[b2][a] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(f.w[b2], f.h[a], acc[b2][a], 0, 0, 0);
            if (u & 1) load_one(st, i0 + (u >> 1));
            __builtin_amdgcn_sched_barrier(0);
        }
    };
    // A tile's accumulators start at 0, except for columns past V (in the
    // last vocabulary tile), which start at -inf: their head rows read as
    // zeros, so they stay -inf and drop out of every statistic without a
    // mask in the fold (the logits mode does not store them).
    auto zero_acc = [&](int v0) {
        if (v0 + kBN <= V) {                         // no column past V: plain zeros
            #pragma unroll
            for (int b2 = 0; b2 < 4; ++b2)
                #pragma unroll
                for (int a = 0; a < 4; ++a) acc[b2][a] = f32x16{};
            return;
        }
        const int lim = V - (v0 + wn * 128 + 4 * (lane >> 5));
        #pragma unroll
        for (int b2 = 0; b2 < 4; ++b2)
            #pragma unroll
            for (int a = 0; a < 4; ++a)
                #pragma unroll
                for (int i = 0; i < 16; ++i)
                    acc[b2][a][i] = 32 * b2 + 8 * (i >> 2) + (i & 3) < lim ? 0.0f : -INFINITY;
    };

    // ---- running statistics of this lane's 4 hidden rows (a: row
    // wm * 128 + 32 a + lane % 32 of the tile) over its columns so far: the
    // maximum and the exp-sum under it (sampled) or the first argmax, and
    // the drafted token's logit where this lane saw it.
    float rm[4], rx[4], rz[4];
    int xt[4];                                       // the rows' drafted tokens (-1: none)
    auto start_band = [&](int r0) {
        #pragma unroll
        for (int a = 0; a < 4; ++a) {
            rm[a] = -INFINITY;
            rx[a] = kSampled ? 0.0f : __int_as_float(INT_MAX);
            rz[a] = NAN;
            const int r = r0 + wm * 128 + 32 * a + (lane & 31);
            xt[a] = (tok && r < R) ? tok[r] : -1;
        }
    };
    // Fold the tile into the running statistics, one 32 x 32 block at a
    // time. A lane's columns of a row go up with (vocabulary block, i):
    // column cbase + 32 b2 + 8 (i / 4) + i % 4, so the first maximum wins.
    // Columns past V hold -inf (see zero_acc).
    auto fold = [&](int v0) {
        const int cbase = v0 + wn * 128 + 4 * (lane >> 5);
        #pragma unroll
        for (int a = 0; a < 4; ++a) {
            // Where the drafted token lies among this lane's columns, if it
            // does: block tb, element ti.
            const unsigned o = (unsigned)(xt[a] - (v0 + wn * 128));
            const bool hit = o < 128u && ((o >> 2) & 1u) == (unsigned)(lane >> 5);
            const int tb = (int)(o >> 5), ti = (int)(((o >> 3) & 3u) * 4u + (o & 3u));
            const bool any_hit = __builtin_amdgcn_ballot_w64(hit) != 0;
            #pragma unroll
            for (int b2 = 0; b2 < 4; ++b2) {
                float z[16];
                #pragma unroll
                for (int i = 0; i < 16; ++i) z[i] = acc[b2][a][i];
                if (any_hit) {
                    #pragma unroll
                    for (int i = 0; i < 16; ++i)
                        if (hit && tb == b2 && ti == i) rz[a] = z[i];
                }
                float mb = z[0];
                #pragma unroll
                for (int i = 1; i < 16; ++i) mb = fmaxf(mb, z[i]);
                if (kSampled) {
                    // A block of -inf (past V) adds nothing. (Taking the
                    // block as a branch also keeps the compiler from
                    // interleaving all 16 blocks' values at once.)
                    if (mb > -INFINITY) {
                        const float mr = fmaxf(rm[a], mb);
                        float sum = 0.0f;
                        #pragma unroll
                        for (int i = 0; i < 16; ++i) sum += __builtin_amdgcn_exp2f((z[i] - mr) * c);
                        rx[a] = rx[a] * __builtin_amdgcn_exp2f((rm[a] - mr) * c) + sum;
                        rm[a] = mr;
                    }
                } else if (mb > rm[a]) {
                    // A new maximum in this block: its first column.
                    int ib = 15;
                    #pragma unroll
                    for (int i = 14; i >= 0; --i) ib = z[i] == mb ? i : ib;
                    rm[a] = mb;
                    rx[a] = __int_as_float(cbase + 32 * b2 + 8 * (ib >> 2) + (ib & 3));
                }
            }
        }
    };

    // Logits: the tile's values to out, 4 consecutive columns per store (16
    // bytes when V is a multiple of 4); rows from R on and columns from V on
    // are not written.
    auto store = [&](int v0, int r0) {
        const int cbase = v0 + wn * 128 + 4 * (lane >> 5);
        const bool vec = (V & 3) == 0;
        #pragma unroll
        for (int a = 0; a < 4; ++a) {
            const int r = r0 + wm * 128 + 32 * a + (lane & 31);
            float* orow = out + (size_t)(r < R ? r : 0) * V;
            #pragma unroll
            for (int b2 = 0; b2 < 4; ++b2)
                #pragma unroll
                for (int q = 0; q < 4; ++q) {
                    const int col = cbase + 32 * b2 + 8 * q;
                    const f32x16& t = acc[b2][a];
                    if (r < R && vec && col + 3 < V) {
                        *reinterpret_cast<float4*>(orow + col) =
                            float4{t[4 * q], t[4 * q + 1], t[4 * q + 2], t[4 * q + 3]};
                    } else if (r < R) {
                        #pragma unroll
                        for (int e = 0; e < 4; ++e)
                            if (col + e < V) orow[col + e] = t[4 * q + e];
                    }
                }
        }
    };

    // Draw masses (kMass). Packed row r is the target row (bit 3 of r clear)
    // or the drafter row of request 8 (r / 16) + r % 8, so in each 32 x 32
    // block the lanes l and l ^ 8 hold a request's two rows over the same
    // columns. Each lane's 4 rows' normalisers are set per row tile.
    float dm_k[4];                                   // the row's exponent offset (mass_offset)
    int dm_b[4];                                     // the row's request (-1: none)
    auto start_mass_rows = [&](int r0) {
        #pragma unroll
        for (int a = 0; a < 4; ++a) {
            const int r = r0 + wm * 128 + 32 * a + (lane & 31);
            const int b = 8 * (r >> 4) + (r & 7);
            dm_b[a] = -1;
            dm_k[a] = INFINITY;                      // a row without mass
            if (b < dm.nreq) {
                const DrawDesc d = dm.desc[b];
                if (d.kind != kNoDraw) {
                    dm_b[a] = b;
                    if (((r >> 3) & 1) == 0) {
                        dm_k[a] = svhead::mass_offset(d.mt, d.st, c);
                    } else if (d.kind == kResidual) {
                        dm_k[a] = svhead::mass_offset(d.md, d.sd, c);
                    }
                }
            }
        }
    };
    // The tile's draw masses: each lane's values 2^(z c - k) of its row
    // (k = mass_offset(m, S, c)), the drafter row's taken from lane ^ 8 (a DPP rotation by 8 within
    // a row of 16 lanes), summed per 4 consecutive columns in fp32 and per
    // half block (16 columns: lanes l < 32 hold columns 0-3, 8-11, 16-19,
    // 24-27 of a 32-column block, lanes l + 32 the others) in fp64. The
    // target row's lanes store both halves; a block's mass is their sum.
    auto mass_fold = [&](int v0) {
        const int nb32 = (V + 31) >> 5;
        const int cw = v0 + wn * 128;
        const bool tgt = ((lane >> 3) & 1) == 0;
        const int half = lane >> 5;
        #pragma unroll
        for (int a = 0; a < 4; ++a) {
            #pragma unroll
            for (int b2 = 0; b2 < 4; ++b2) {
                double sr = 0.0, sp = 0.0;
                #pragma unroll
                for (int g = 0; g < 4; ++g) {
                    float r4 = 0.0f, p4 = 0.0f;
                    #pragma unroll
                    for (int t = 0; t < 4; ++t) {
                        const float pv =
                            __builtin_amdgcn_exp2f(__builtin_fmaf(acc[b2][a][4 * g + t], c, -dm_k[a]));
                        const float qv = __int_as_float(__builtin_amdgcn_mov_dpp(
                            __float_as_int(pv), 0x128, 0xF, 0xF, false));   // row_ror:8
                        const float rv = fmaxf(pv - qv, 0.0f);
                        r4 = t ? r4 + rv : rv;
                        p4 = t ? p4 + pv : pv;
                    }
                    sr += (double)r4;
                    sp += (double)p4;
                }
                const int col = cw + 32 * b2;
                if (tgt && dm_b[a] >= 0 && col < V) {
                    const size_t at = ((size_t)dm_b[a] * (size_t)nb32 + (size_t)(col >> 5)) * 2 + half;
                    dm.mres[at] = sr;
                    dm.mp[at] = sp;
                }
            }
        }
    };

    // The band's partial of this (XCD, column slot) for each of its rows:
    // the lane pair holding a row (lane, lane ^ 32) merges, then the two
    // waves with the same rows through LDS.
    auto flush = [&](int r0, int ps) {
        #pragma unroll
        for (int a = 0; a < 4; ++a) {
            float m2 = __shfl_xor(rm[a], 32, 64), x2 = __shfl_xor(rx[a], 32, 64);
            const float z2 = __shfl_xor(rz[a], 32, 64);
            if (kSampled) {
                merge_ms(rm[a], rx[a], m2, x2, c, true);
            } else {
                int ai = __float_as_int(rx[a]);
                merge_arg(rm[a], ai, m2, __float_as_int(x2));
                rx[a] = __int_as_float(ai);
            }
            if (rz[a] != rz[a]) rz[a] = z2;
        }
        const int rl0 = wm * 128 + (lane & 31);
        if (wn == 1 && lane < 32) {
            #pragma unroll
            for (int a = 0; a < 4; ++a) {
                xw[rl0 + 32 * a] = HeadPart{rm[a], kSampled ? rx[a] : 0.0f, rz[a],
                                            kSampled ? INT_MAX : __float_as_int(rx[a])};
            }
        }
        __syncthreads();
        if (wn == 0 && lane < 32) {
            #pragma unroll
            for (int a = 0; a < 4; ++a) {
                const int rl = rl0 + 32 * a;
                const HeadPart o = xw[rl];
                HeadPart o2;
                o2.m = rm[a];
                o2.zx = rz[a] == rz[a] ? rz[a] : o.zx;
                if (kSampled) {
                    o2.s = rx[a];
                    merge_ms(o2.m, o2.s, o.m, o.s, c, true);
                    o2.arg = INT_MAX;
                } else {
                    o2.s = 0.0f;
                    o2.arg = __float_as_int(rx[a]);
                    merge_arg(o2.m, o2.arg, o.m, o.arg);
                }
                if (r0 + rl < R) part[(size_t)ps * R + r0 + rl] = o2;
            }
        }
        __syncthreads();
    };

    // ---- the stream. Step g (tile c_stp, k-step ks) lives in stage g % 2.
    // Its 64 of k are multiplied as four groups of 16, each group's
    // fragments read while the previous group is multiplied. Before the
    // last group the workgroup synchronises (step g + 1 has landed, and every
    // wave has read step g into registers), reads step g + 1's first group
    // and starts refilling stage g % 2 with step g + 2: half of its loads go
    // out among the last group's products, half among the first group's
    // products of step g + 1. Tiles follow one another without a pause; a
    // tile's statistics are folded after its last product.
    int c_stp = next_tile(side ? t_beg : xcd);
    if (c_stp >= total) return;                      // (a side workgroup without tiles)
    loader_at(c_stp);
    #pragma unroll
    for (int i = 0; i < 16; ++i) load_one(0, i);     // step 0, whole
    loader_next();
    int band = band_of(c_stp);
    if (kRowStats) start_band(row0_of(c_stp));
    if (kMass) start_mass_rows(row0_of(c_stp));
    zero_acc(v0_of(c_stp));
    __builtin_amdgcn_s_waitcnt(0);                   // step 0 and the tokens
    ring_barrier();
    Frags f0, f1;
    read_frags(f0, 0, 0);
    if (l_stp < total) {
        #pragma unroll
        for (int i = 0; i < 8; ++i) load_one(1, i);  // step 1, first half
    }
    int st = 0;
    for (;;) {
        // Steps 0 .. nk - 2 of the tile: the next step is in this tile.
        for (int ks = 0; ks + 1 < nk; ++ks) {
            read_frags(f1, st, 1);
            __builtin_amdgcn_sched_barrier(0);
            multiply_ld(f0, st ^ 1, 8);              // step g + 1, second half
            loader_next();                           // the loader moves on to step g + 2
            read_frags(f0, st, 2);
            __builtin_amdgcn_sched_barrier(0);
            multiply(f1);
            __builtin_amdgcn_sched_barrier(0);
            read_frags(f1, st, 3);
            __builtin_amdgcn_sched_barrier(0);
            multiply(f0);
            __builtin_amdgcn_sched_barrier(0);
            wait_vm<0>();                            // this wave's loads of step g + 1
            ring_barrier();                          // everyone's; step g read by all
            read_frags(f0, st ^ 1, 0);
            __builtin_amdgcn_sched_barrier(0);
            multiply_ld(f1, st, 0);                  // step g + 2, first half
            __builtin_amdgcn_sched_barrier(0);
            st ^= 1;
        }
        // The tile's last step; the next step, if any, starts the next tile
        // (its first group is read after the fold). The synchronisation
        // happens even when nothing follows: the loads among the last
        // group's products then refill the stage this step used.
        const int n_stp = next_tile(c_stp + stride);
        const bool has_next = n_stp < total;
        read_frags(f1, st, 1);
        __builtin_amdgcn_sched_barrier(0);
        multiply_ld(f0, st ^ 1, 8);
        loader_next();
        read_frags(f0, st, 2);
        __builtin_amdgcn_sched_barrier(0);
        multiply(f1);
        __builtin_amdgcn_sched_barrier(0);
        read_frags(f1, st, 3);
        __builtin_amdgcn_sched_barrier(0);
        multiply(f0);
        __builtin_amdgcn_sched_barrier(0);
        wait_vm<0>();
        ring_barrier();
        __builtin_amdgcn_sched_barrier(0);
        multiply_ld(f1, st, 0);
        __builtin_amdgcn_sched_barrier(0);
        st ^= 1;
        if (kLogits) store(v0_of(c_stp), row0_of(c_stp));
        else if (kMass) mass_fold(v0_of(c_stp));
        else fold(v0_of(c_stp));
        if (!has_next) break;
        const int nb = band_of(n_stp);
        if (kRowStats && nb != band) {
            flush(row0_of(c_stp), pslot_of(c_stp));
            start_band(row0_of(n_stp));
        }
        if (kMass && nb != band) start_mass_rows(row0_of(n_stp));
        band = nb;
        zero_acc(v0_of(n_stp));
        read_frags(f0, st, 0);                       // the next tile's first group
        c_stp = n_stp;
    }
    if (kRowStats) flush(row0_of(c_stp), pslot_of(c_stp));
    __builtin_amdgcn_s_waitcnt(0);                   // the last loads and stores
}

// Per row: merge the splits' partials (in split order) into the outputs.
// Greedy partials carry the first argmax; sampled ones do not (INT_MAX), and
// the sampled call reports none.
// parts > 0: that many partials per row; parts < 0: the many-row product's
// (its super-tile slots and its side columns'); 0: one per vocabulary split
// of the product above.
__global__ void head_merge_kernel(const HeadPart* __restrict__ part, int r_max,
                                  const int* __restrict__ d_rows, int V, float c, int sampled,
                                  int parts, float* out_max, float* out_sum, float* out_z,
                                  int32_t* out_arg) {
    const int R = rows_now(r_max, d_rows);
    const int splits = parts > 0   ? parts
                       : parts < 0 ? kMmParts + mm_split<kBandTiles, kColTiles>(R, V).side_cols
                                   : splits_for(R, V);
    const int r = blockIdx.x * blockDim.x + threadIdx.x;
    if (r >= R) return;
    float m = -INFINITY, s = 0.0f, z = NAN, bv = -INFINITY;
    int ai = INT_MAX;
    // Eight partials' loads in flight at a time; merged in split order.
    constexpr int kBatch = 8;
    for (int sp0 = 0; sp0 < splits; sp0 += kBatch) {
        HeadPart ob[kBatch];
        #pragma unroll
        for (int k = 0; k < kBatch; ++k)
            if (sp0 + k < splits) ob[k] = part[(size_t)(sp0 + k) * R + r];
        #pragma unroll
        for (int k = 0; k < kBatch; ++k) {
            if (sp0 + k >= splits) break;
            const HeadPart& o = ob[k];
            if (sampled) merge_ms(m, s, o.m, o.s, c, true);
            else merge_arg(bv, ai, o.m, o.arg);
            if (z != z) z = o.zx;
        }
    }
    out_max[r] = sampled ? m : bv;
    if (out_sum) out_sum[r] = sampled ? s : NAN;
    if (out_z) out_z[r] = z;
    if (out_arg) out_arg[r] = sampled ? -1 : (ai == INT_MAX ? 0 : ai);
}

bool aligned_to(const void* p, size_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

int items_for(int R, int V) { return ((R + kTM - 1) / kTM) * splits_for(R, V); }

}  // namespace

// The many-row product's instantiations may use more than the default
// dynamic LDS: raised once per process (a thread-safe static).
static hipError_t mm_attrs() {
    static const hipError_t rc = []() {
        const void* fns[] = {
            reinterpret_cast<const void*>(&head_mm_kernel<kMmSampled, kBandTiles, kColTiles>),
            reinterpret_cast<const void*>(&head_mm_kernel<kMmGreedy, kBandTiles, kColTiles>),
            reinterpret_cast<const void*>(&head_mm_kernel<kMmLogits, kLogBand, kLogCols>),
            reinterpret_cast<const void*>(&head_mm_kernel<kMmMass, kLogBand, kLogCols>)};
        for (const void* f : fns) {
            const hipError_t e =
                hipFuncSetAttribute(f, hipFuncAttributeMaxDynamicSharedMemorySize, kMmLds);
            if (e != hipSuccess) return e;
        }
        return hipSuccess;
    }();
    return rc;
}

namespace svhead {

// splits(R) * R stays within max(65536, R) (one resident wave of 128-row
// tiles, or a single split) and within cap * R.
size_t stats_workspace_bytes(int r_max, int V) {
    if (r_max < 1 || V < 1) return 0;
    const long long cap = ((V + kTN - 1) / kTN + 7) / 8;
    long long n = (long long)kResidentSlots * kTM;
    if (r_max > n) n = r_max;
    if (cap * r_max < n) n = cap * r_max;
    // The many-row product (whatever H is): kMmParts partials per row and
    // one per side column.
    const long long mm = (long long)(kMmParts + mm_side_max(V)) * r_max;
    if (mm_shape(r_max, V) && n < mm) n = mm;
    return (size_t)n * sizeof(HeadPart);
}

int head_stats_launch(const HeadRows& rows, const uint16_t* weight, int r_max,
                      const int* d_rows, int H, int V, const int32_t* tokens,
                      float temperature, float* out_max, float* out_sum, float* out_z,
                      int32_t* out_arg, void* workspace, hipStream_t s) {
    if (r_max < 1) return SV_OK;
    const bool sampled = temperature > 0.0f;
    const float c = sampled ? (float)(1.4426950408889634 / (double)temperature) : 0.0f;
    HeadPart* part = static_cast<HeadPart*>(workspace);
    if (mm_path<kBandTiles, kColTiles>(rows, r_max, H, V)) {
        // Many rows: the large-tile product, one workgroup per CU.
        if (mm_attrs() != hipSuccess) return SV_ERR_HIP;
        if (sampled) {
            hipLaunchKernelGGL((head_mm_kernel<kMmSampled, kBandTiles, kColTiles>), dim3(kMmGrid),
                               dim3(kMmThreads), kMmLds, s, rows, weight, r_max, d_rows, H, V,
                               tokens, c, part, nullptr, DrawMass{});
        } else {
            hipLaunchKernelGGL((head_mm_kernel<kMmGreedy, kBandTiles, kColTiles>), dim3(kMmGrid),
                               dim3(kMmThreads), kMmLds, s, rows, weight, r_max, d_rows, H, V,
                               tokens, c, part, nullptr, DrawMass{});
        }
        if (hipGetLastError() != hipSuccess) return SV_ERR_HIP;
        hipLaunchKernelGGL(head_merge_kernel, dim3((unsigned)((r_max + 255) / 256)), dim3(256), 0,
                           s, part, r_max, d_rows, V, c, sampled ? 1 : 0, -1, out_max,
                           out_sum, out_z, out_arg);
        return hipGetLastError() == hipSuccess ? SV_OK : SV_ERR_HIP;
    }
    // One workgroup per item. With the count read on the device, the grid
    // covers every count up to r_max: up to 512 row tiles a count has at most
    // 512 items, beyond that one split, so no more items than r_max has.
    int grid = items_for(r_max, V);
    if (d_rows && grid < kResidentSlots) grid = kResidentSlots;
    if (sampled) {
        hipLaunchKernelGGL(head_stats_kernel<kEpiSampled>, dim3((unsigned)grid),
                           dim3(kHThreads), 0, s, rows, weight, r_max, d_rows, H, V, tokens, c,
                           part, nullptr, RowAdd{});
    } else {
        hipLaunchKernelGGL(head_stats_kernel<kEpiGreedy>, dim3((unsigned)grid),
                           dim3(kHThreads), 0, s, rows, weight, r_max, d_rows, H, V, tokens, c,
                           part, nullptr, RowAdd{});
    }
    if (hipGetLastError() != hipSuccess) return SV_ERR_HIP;
    hipLaunchKernelGGL(head_merge_kernel, dim3((unsigned)((r_max + 255) / 256)), dim3(256), 0, s,
                       part, r_max, d_rows, V, c, sampled ? 1 : 0, 0, out_max, out_sum, out_z,
                       out_arg);
    return hipGetLastError() == hipSuccess ? SV_OK : SV_ERR_HIP;
}

int head_logits_launch(const HeadRows& rows, const uint16_t* weight, int R, int H, int V,
                       float* out, hipStream_t s) {
    if (R < 1) return SV_OK;
    if (mm_path<kLogBand, kLogCols>(rows, R, H, V)) {
        if (mm_attrs() != hipSuccess) return SV_ERR_HIP;
        hipLaunchKernelGGL((head_mm_kernel<kMmLogits, kLogBand, kLogCols>), dim3(kMmGrid),
                           dim3(kMmThreads), kMmLds, s, rows, weight, R, nullptr, H, V, nullptr,
                           0.0f, nullptr, out, DrawMass{});
        return hipGetLastError() == hipSuccess ? SV_OK : SV_ERR_HIP;
    }
    hipLaunchKernelGGL(head_stats_kernel<kEpiLogits>, dim3((unsigned)items_for(R, V)),
                       dim3(kHThreads), 0, s, rows, weight, R, nullptr, H, V, nullptr, 0.0f,
                       nullptr, out, RowAdd{});
    return hipGetLastError() == hipSuccess ? SV_OK : SV_ERR_HIP;
}

bool mass_path(const HeadRows& rows, int R, int H, int V) {
    return R >= 1 && mm_path<kLogBand, kLogCols>(rows, R, H, V);
}

int head_mass_launch(const HeadRows& rows, const uint16_t* weight, int R, int H, int V, float c,
                     const DrawMass& dm, hipStream_t s) {
    if (!mass_path(rows, R, H, V)) return SV_ERR_ARG;
    if (mm_attrs() != hipSuccess) return SV_ERR_HIP;
    hipLaunchKernelGGL((head_mm_kernel<kMmMass, kLogBand, kLogCols>), dim3(kMmGrid),
                       dim3(kMmThreads), kMmLds, s, rows, weight, R, nullptr, H, V, nullptr, c,
                       nullptr, nullptr, dm);
    return hipGetLastError() == hipSuccess ? SV_OK : SV_ERR_HIP;
}

int add_splits(int R, int V) { return splits_for(R, V); }

int head_add_bf16_launch(const HeadRows& rows, const uint16_t* weight, int R, int H, int V,
                         const uint16_t* base, uint16_t* out, long long row_stride,
                         ArgPart* arg, hipStream_t s) {
    if (R < 1) return SV_OK;
    hipLaunchKernelGGL(head_stats_kernel<kEpiAddBf16>, dim3((unsigned)items_for(R, V)),
                       dim3(kHThreads), 0, s, rows, weight, R, nullptr, H, V, nullptr, 0.0f,
                       nullptr, nullptr, RowAdd{base, out, row_stride, arg});
    return hipGetLastError() == hipSuccess ? SV_OK : SV_ERR_HIP;
}

}  // namespace svhead

extern "C" size_t spec_head_workspace_bytes(int R, int V) {
    if (R < 1 || V < 1) return 0;
    size_t n = (size_t)splits_for(R, V) * (size_t)R;
    const size_t mm = (size_t)(kMmParts + mm_side_max(V)) * (size_t)R;
    if (mm_shape(R, V) && n < mm) n = mm;
    return n * sizeof(HeadPart);
}

extern "C" int spec_head_stats(const void* hidden, const void* weight, int R, int H, int V,
                               const int32_t* tokens, float temperature, float* out_max,
                               float* out_sumexp, float* out_ztok, int32_t* out_argmax,
                               void* workspace, size_t workspace_bytes, void* stream) {
    if (R < 0 || H < 1 || V < 1 || V > SV_MAX_VOCAB || (H % 8) != 0 ||
        !std::isfinite(temperature) || temperature < 0.0f) {
        return SV_ERR_ARG;
    }
    if (R == 0) return SV_OK;
    if (!hidden || !weight || !out_max || !workspace) return SV_ERR_NULL;
    if (!aligned_to(hidden, 16) || !aligned_to(weight, 16) || !aligned_to(out_max, 4) ||
        (out_sumexp && !aligned_to(out_sumexp, 4)) || (out_ztok && !aligned_to(out_ztok, 4)) ||
        (out_argmax && !aligned_to(out_argmax, 4)) || (tokens && !aligned_to(tokens, 4)) ||
        !aligned_to(workspace, 16)) {
        return SV_ERR_ALIGN;
    }
    if (workspace_bytes < spec_head_workspace_bytes(R, V)) return SV_ERR_ARG;
    const HeadRows rows{static_cast<const uint16_t*>(hidden), nullptr, nullptr, R, 0};
    return svhead::head_stats_launch(rows, static_cast<const uint16_t*>(weight), R, nullptr, H,
                                     V, tokens, temperature, out_max, out_sumexp, out_ztok,
                                     out_argmax, workspace, static_cast<hipStream_t>(stream));
}
