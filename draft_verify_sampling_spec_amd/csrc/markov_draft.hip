// markov_draft.hip -- the drafter's low-rank Markov head over a drafted
// block, for MI355X (gfx950).
//
// What is computed: "Speculative decoding becomes standard: DSpark and
// multi-token drafters", section "What DSpark adds", paragraph 1 (the block
// comes from a parallel backbone, and a light sequential correction, a
// factorised rank-256 Markov model over consecutive positions, keeps the
// block consistent), and the "DSpark" finds page's comparison of its two
// sequential structures (the deployed one conditions only on the preceding
// token, through a low-rank matrix). Reading: drafted position i's logits are the backbone's
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
//      memory. The same epilogue follows the values it stores with a first
//      argmax per row and vocabulary split;
//   2. one wave per request merges its splits' argmaxes (ties to the lower
//      column): the first argmax of the stored row, which is x_i and the
//      next position's row map (two map buffers alternate). The stored rows
//      are not read back.
// A seed launch checks the given last tokens and writes the first row map.

#include <hip/hip_runtime.h>

#include <climits>
#include <cmath>
#include <cstdint>

#include "head_gemm.h"
#include "spec_verify.h"

namespace {

using svhead::ArgPart;
using svhead::HeadRows;

constexpr int kMkPickThreads = 256;
constexpr int kMkPickWaves = kMkPickThreads / 64;     // one request per wave

struct MkLayout {
    size_t map0, map1, parts, total;
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
    L.map0 = take((size_t)B * 4);
    L.map1 = take((size_t)B * 4);
    L.parts = take((size_t)svhead::add_splits(B, V) * (size_t)B * sizeof(ArgPart));
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

__device__ __forceinline__ bool mk_better(float v, int i, float bv, int bi) {
    return v > bv || (v == bv && i < bi);
}

// Position i's token of each request, one wave per request: the first
// argmax over its splits' entries. A larger value wins, an equal one only
// from a lower column; columns are unique, so the result does not depend on
// the order of the merges, and the lanes take the splits in parallel.
__global__ __launch_bounds__(kMkPickThreads) void mk_pick_kernel(
    const ArgPart* __restrict__ part, int splits, int B, int K, int V, int i,
    int32_t* __restrict__ out_tokens, int32_t* __restrict__ next_map) {
    const int lane = threadIdx.x & 63;
    const int b = blockIdx.x * kMkPickWaves + (int)(threadIdx.x >> 6);
    if (b >= B) return;                                // whole waves leave together
    float bv = -INFINITY;
    int bi = INT_MAX;
    for (int sp = lane; sp < splits; sp += 64) {
        const ArgPart a = part[(size_t)sp * B + b];
        if (mk_better(a.v, a.i, bv, bi)) {
            bv = a.v;
            bi = a.i;
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
        const int x = (bi >= 0 && bi < V) ? bi : 0;   // no value above -inf: token 0
        out_tokens[(size_t)b * K + i] = x;
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
    ArgPart* parts = reinterpret_cast<ArgPart*>(ws + L.parts);
    const int splits = svhead::add_splits(B, V);
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
        const HeadRows rows{A, nullptr, map[i & 1], V, 0};
        const int rc = svhead::head_add_bf16_launch(rows, Bm, B, r, V, base + (size_t)i * V,
                                                    out + (size_t)i * V, (long long)K * V, parts,
                                                    s);
        if (rc != SV_OK) return rc;
        hipLaunchKernelGGL(mk_pick_kernel, dim3((unsigned)((B + kMkPickWaves - 1) / kMkPickWaves)),
                           dim3(kMkPickThreads), 0, s, parts, splits, B, K, V, i, out_tokens,
                           map[(i + 1) & 1]);
        if (hipGetLastError() != hipSuccess) return SV_ERR_HIP;
    }
    return SV_OK;
}
