// markov_draft.hip -- the drafter's low-rank Markov head over a drafted
// block, for MI355X (gfx950).
//
// What is computed: "Speculative decoding becomes standard: DSpark and
// multi-token drafters", section "What DSpark adds", paragraph 1 (a parallel
// backbone proposes a block of tokens and a small sequential head, a
// low-rank Markov module of rank 256, models the dependencies between the
// block's positions), and the "DSpark" finds page's list of the two
// sequential structures (the Markov head uses only the previous token and a
// low-rank matrix). Reading: drafted position i's logits are the backbone's
// row plus row x_{i-1} of the factored transition matrix A Bm^T (A, Bm are
// [V, r]); the row is stored as bf16 and the drafted token x_i is its first
// argmax; x_{-1} is the last token already in each sequence.
//
// Design, per drafted position i (two stream-ordered launches; positions run
// in order because x_i feeds position i+1):
//   1. the matrix cores form the bias A[x_{i-1}[b]] Bm^T in fp32 -- the
//      output head's product with the previous tokens as its row map and the
//      rank r as its depth -- and its epilogue stages each output tile in
//      LDS: the backbone values come in with 16-byte loads, each bias is
//      added in fp32 and rounded once to bf16 (to nearest, ties to even), and
//      the drafter rows go out with 16-byte stores, so the bias never reaches
//      memory;
//   2. one workgroup per request reads its stored row back and takes the
//      first argmax, which is x_i and the next position's row map (two map
//      buffers alternate).
// A seed launch checks the given last tokens and writes the first row map.

#include <hip/hip_runtime.h>

#include <climits>
#include <cmath>
#include <cstdint>

#include "head_gemm.h"
#include "spec_verify.h"

namespace {

using svhead::HeadRows;

constexpr int kMkThreads = 512;                    // 8 waves per request row
constexpr int kMkGroup = 8;                        // elements per lane per step (16 B of bf16)
constexpr int kMkUnroll = 2;                       // groups in flight per lane

struct MkLayout {
    size_t map0, map1, total;
};

size_t mk_up256(size_t x) { return (x + 255) & ~(size_t)255; }

MkLayout mk_layout(int B, int V) {
    MkLayout L{};
    size_t o = 0;
    auto take = [&](size_t bytes) {
        const size_t at = o;
        o += mk_up256(bytes);
        return at;
    };
    (void)V;
    L.map0 = take((size_t)B * 4);
    L.map1 = take((size_t)B * 4);
    L.total = o;
    return L;
}

// The first row map: the given last tokens; one outside [0, V) becomes -1 (a
// row of zeros in the product) and raises SV_FLAG_BAD_TOKEN.
__global__ void mk_seed_kernel(const int32_t* __restrict__ prev, int B, int V,
                               int32_t* __restrict__ map, int32_t* __restrict__ status) {
    __shared__ int bad;
    if (threadIdx.x == 0) bad = 0;
    __syncthreads();
    int mine = 0;
    for (int b = threadIdx.x; b < B; b += blockDim.x) {
        const int t = prev[b];
        const bool ok = t >= 0 && t < V;
        map[b] = ok ? t : -1;
        mine |= ok ? 0 : 1;
    }
    if (mine) atomicOr(&bad, 1);
    __syncthreads();
    if (threadIdx.x == 0 && status) status[0] = bad ? (int32_t)SV_FLAG_BAD_TOKEN : 0;
}

__device__ __forceinline__ float bf16_value(uint32_t bits16) {
    return __uint_as_float(bits16 << 16);
}

__device__ __forceinline__ bool mk_better(float v, int i, float bv, int bi) {
    return v > bv || (v == bv && i < bi);
}

// The first argmax of one stored request row of position i: x_i, written to
// the drafted tokens and the next position's row map. kVec: 16-byte loads
// are legal (V % 8 == 0).
template <bool kVec>
__global__ __launch_bounds__(kMkThreads) void mk_argmax_kernel(
    const uint16_t* __restrict__ z, int K, int V, int i, int32_t* __restrict__ out_tokens,
    int32_t* __restrict__ next_map) {
    __shared__ float wv[kMkThreads / 64];
    __shared__ int wi[kMkThreads / 64];
    const int b = blockIdx.x;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const size_t row = (size_t)b * K + i;
    const uint16_t* src = z + row * (size_t)V;
    float bv = -INFINITY;
    int bi = INT_MAX;
    constexpr int step = kMkThreads * kMkGroup;
    if (kVec) {
        for (int e0 = tid * kMkGroup; e0 < V; e0 += step * kMkUnroll) {
            uint4 g[kMkUnroll];
            #pragma unroll
            for (int u = 0; u < kMkUnroll; ++u) {
                const int e = e0 + u * step;
                if (e < V) g[u] = *reinterpret_cast<const uint4*>(src + e);
            }
            #pragma unroll
            for (int u = 0; u < kMkUnroll; ++u) {
                const int e = e0 + u * step;
                if (e < V) {
                    const uint32_t w[4] = {g[u].x, g[u].y, g[u].z, g[u].w};
                    #pragma unroll
                    for (int k = 0; k < 4; ++k) {
                        const float vl = bf16_value(w[k] & 0xFFFFu), vh = bf16_value(w[k] >> 16);
                        if (vl > bv) {              // a lane's elements go up in index order
                            bv = vl;
                            bi = e + 2 * k;
                        }
                        if (vh > bv) {
                            bv = vh;
                            bi = e + 2 * k + 1;
                        }
                    }
                }
            }
        }
    } else {
        for (int e0 = tid * kMkGroup; e0 < V; e0 += step) {
            #pragma unroll
            for (int k = 0; k < kMkGroup; ++k) {
                const int e = e0 + k;
                if (e < V) {
                    const float v = bf16_value(src[e]);
                    if (v > bv) {
                        bv = v;
                        bi = e;
                    }
                }
            }
        }
    }
    #pragma unroll
    for (int o = 32; o > 0; o >>= 1) {
        const float ov = __shfl_xor(bv, o, 64);
        const int oi = __shfl_xor(bi, o, 64);
        if (mk_better(ov, oi, bv, bi)) {
            bv = ov;
            bi = oi;
        }
    }
    if (lane == 0) {
        wv[wave] = bv;
        wi[wave] = bi;
    }
    __syncthreads();
    if (tid == 0) {
        for (int w = 1; w < kMkThreads / 64; ++w) {
            if (mk_better(wv[w], wi[w], bv, bi)) {
                bv = wv[w];
                bi = wi[w];
            }
        }
        const int x = (bi >= 0 && bi < V) ? bi : 0;   // an all-NaN row (undefined input)
        out_tokens[row] = x;
        next_map[b] = x;
    }
}

bool mk_aligned(const void* p, size_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

}  // namespace

extern "C" size_t spec_markov_draft_workspace_bytes(int B, int V) {
    if (B < 1 || B > SV_MAX_BATCH || V < 1 || V > SV_MAX_VOCAB) return 0;
    return mk_layout(B, V).total;
}

extern "C" int spec_markov_draft(const void* base_logits, const void* markov_a,
                                 const void* markov_b, const int32_t* prev_tokens, int B, int K,
                                 int r, int V, void* out_logits, int32_t* out_tokens,
                                 int32_t* out_status, void* workspace, size_t workspace_bytes,
                                 void* stream) {
    if (B < 0 || B > SV_MAX_BATCH || K < 0 || K > SV_MAX_K || r < 8 || (r % 8) != 0 || V < 1 ||
        V > SV_MAX_VOCAB) {
        return SV_ERR_ARG;
    }
    if (B == 0 || K == 0) return SV_OK;
    if (!base_logits || !markov_a || !markov_b || !prev_tokens || !out_logits || !out_tokens ||
        !workspace) {
        return SV_ERR_NULL;
    }
    if (!mk_aligned(base_logits, 16) || !mk_aligned(markov_a, 16) || !mk_aligned(markov_b, 16) ||
        !mk_aligned(out_logits, 16) || !mk_aligned(prev_tokens, 4) || !mk_aligned(out_tokens, 4) ||
        (out_status && !mk_aligned(out_status, 4)) || !mk_aligned(workspace, 256)) {
        return SV_ERR_ALIGN;
    }
    if (base_logits == out_logits) return SV_ERR_ARG;
    const MkLayout L = mk_layout(B, V);
    if (workspace_bytes < L.total) return SV_ERR_ARG;
    char* ws = static_cast<char*>(workspace);
    int32_t* map[2] = {reinterpret_cast<int32_t*>(ws + L.map0),
                       reinterpret_cast<int32_t*>(ws + L.map1)};
    const hipStream_t s = static_cast<hipStream_t>(stream);
    const uint16_t* A = static_cast<const uint16_t*>(markov_a);
    const uint16_t* Bm = static_cast<const uint16_t*>(markov_b);
    const uint16_t* base = static_cast<const uint16_t*>(base_logits);
    uint16_t* out = static_cast<uint16_t*>(out_logits);

    hipLaunchKernelGGL(mk_seed_kernel, dim3(1), dim3(1024), 0, s, prev_tokens, B, V, map[0],
                       out_status);
    if (hipGetLastError() != hipSuccess) return SV_ERR_HIP;
    for (int i = 0; i < K; ++i) {
        // Rows of A indexed by the previous tokens; virtual rows >= V never
        // occur (tokens are checked, argmaxes lie in [0, V)).
        const HeadRows rows{A, nullptr, map[i & 1], V};
        const int rc = svhead::head_add_bf16_launch(rows, Bm, B, r, V, base + (size_t)i * V,
                                                    out + (size_t)i * V, (long long)K * V, s);
        if (rc != SV_OK) return rc;
        if (V % kMkGroup == 0) {
            hipLaunchKernelGGL(mk_argmax_kernel<true>, dim3((unsigned)B), dim3(kMkThreads), 0, s, out,
                               K, V, i, out_tokens, map[(i + 1) & 1]);
        } else {
            hipLaunchKernelGGL(mk_argmax_kernel<false>, dim3((unsigned)B), dim3(kMkThreads), 0, s,
                               out, K, V, i, out_tokens, map[(i + 1) & 1]);
        }
        if (hipGetLastError() != hipSuccess) return SV_ERR_HIP;
    }
    return SV_OK;
}
