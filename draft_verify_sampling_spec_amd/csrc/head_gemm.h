// head_gemm.h -- internal interface of the output-head matrix product
// (head_stats.hip) for the other translation units of the library. Not part
// of the C ABI.
//
// The product z = h W^T of bf16 hidden states and the shared head runs on the
// matrix cores with one of five epilogues: per-row statistics for sampled or
// greedy verification, the fp32 logits themselves for a few rows, the draw
// masses of paired target and drafter rows, or the logits added to bf16 rows
// and stored rounded (the Markov head's transition term on the backbone's
// logits). Every epilogue accumulates each logit in
// the same order, so the logits written for a row equal, bit for bit, the
// values its statistics were taken over.
#pragma once

#include <hip/hip_runtime.h>

#include <cmath>
#include <cstddef>
#include <cstdint>

namespace svhead {

// Where the hidden state of packed row r lives. Virtual rows [0, a_rows)
// are rows of `a`, virtual rows [a_rows, a_rows + b_rows) rows of `b`.
// `map` turns packed rows into virtual rows (NULL: identity); a negative
// entry is a row of zeros whose outputs nobody reads. grouped8: the packed
// rows 8i .. 8i + 7 never mix rows of a and rows of b (the many-row product
// needs this when b has rows).
struct HeadRows {
    const uint16_t* a;
    const uint16_t* b;
    const int32_t* map;
    int a_rows;
    int b_rows;
    bool grouped8;
};

// One request's draw in the verify step from hidden states: the normalisers
// of its draw rows, the sampling uniform, and what is drawn.
enum DrawKind { kNoDraw = 0, kResidual = 1, kBonus = 2 };
struct DrawDesc {
    float mt, st;   // target row: max, exp-sum
    float md, sd;   // drafter row (a residual)
    float u;        // the sampling uniform of the drawn position
    int kind;       // DrawKind
    int pos;        // output position j_b
    int pad;
};

// The exponent offset of a draw row's masses: a value's mass is
// 2^(z c - k) with k = m c + log2(S) (m the row's maximum, S its exp-sum
// under m, c = log2(e) / T), k formed in fp64 and rounded once, so that
// 2^(z c - k) = 2^((z - m) c) / S up to that rounding and the exp2's.
__host__ __device__ inline float mass_offset(float m, float S, float c) {
    return (float)((double)m * (double)c + log2((double)S));
}

// Draw masses of the draw rows, per request and block of 32 vocabulary
// columns (block v / 32, ceil(V / 32) blocks per request), in two halves
// (entry 2 (b nb + block) + h, h = 0 for columns 0-3, 8-11, 16-19, 24-27 of
// the block, 1 for the others): the residual max(0, p - q) in mres and p
// alone in mp, each half the fp64 sum of four fp32 sums of 4 consecutive
// columns. p(v) = 2^(z_t(v) c - mass_offset(mt, st, c)), and q(v) likewise
// from the drafter row (0 for a bonus draw).
struct DrawMass {
    const DrawDesc* desc;
    double* mres;
    double* mp;
    int nreq;
};

// Scratch (bytes) for head_stats_launch with at most r_max rows.
size_t stats_workspace_bytes(int r_max, int V);

// `weight` is the head, bf16 [V, H] row-major. H is a multiple of 8 and
// every pointer 16-byte aligned (the callers check).
//
// Row statistics of packed rows [0, R), R = min(*d_rows, r_max) read on the
// device when d_rows is non-NULL, else R = r_max. Outputs as spec_head_stats
// (out_max [R]; out_sum, out_z, out_arg [R] or NULL); temperature == 0 gives
// the greedy statistics. Returns an sv_status code.
int head_stats_launch(const HeadRows& rows, const uint16_t* weight, int r_max,
                      const int* d_rows, int H, int V, const int32_t* tokens,
                      float temperature, float* out_max, float* out_sum, float* out_z,
                      int32_t* out_arg, void* workspace, hipStream_t stream);

// fp32 logits of packed rows [0, R) into out [R, V] (rows whose map entry is
// negative are not written). Returns an sv_status code.
int head_logits_launch(const HeadRows& rows, const uint16_t* weight, int R, int H, int V,
                       float* out, hipStream_t stream);

// One row's first argmax over one vocabulary split of the add-and-store
// product: the largest stored value and the lowest column holding it
// (v = -inf, i = INT_MAX: no column of the split holds a value above -inf).
struct ArgPart {
    float v;
    int i;
};

// Vocabulary splits of head_add_bf16_launch for R rows; split s covers
// columns below those of split s + 1.
int add_splits(int R, int V);

// Whether head_mass_launch takes R packed rows (the many-row product's
// shape and layout conditions).
bool mass_path(const HeadRows& rows, int R, int H, int V);

// The draw masses of R packed draw rows: rows 16g .. 16g + 7 are the target
// rows of requests 8g .. 8g + 7 and rows 16g + 8 .. 16g + 15 their drafter
// rows (a negative map entry: a row of zeros). The logits themselves are not
// written. c = log2(e) / T. Returns SV_ERR_ARG when !mass_path(rows, R, H, V).
int head_mass_launch(const HeadRows& rows, const uint16_t* weight, int R, int H, int V, float c,
                     const DrawMass& dm, hipStream_t stream);

// Logits of packed rows [0, R) added to bf16 rows: for row r and column v,
// out[r * row_stride + v] = bf16(base[r * row_stride + v] + z[r, v]), the sum
// in fp32 and one rounding to nearest even (a row whose map entry is
// negative has z = 0). The tile is staged in LDS so that global loads and
// stores are 16 bytes wide when V is a multiple of 8. With arg non-NULL
// ([add_splits(R, V)][R]), each (split, row) also gets the first argmax of
// the values stored there. Returns an sv_status code.
int head_add_bf16_launch(const HeadRows& rows, const uint16_t* weight, int R, int H, int V,
                         const uint16_t* base, uint16_t* out, long long row_stride,
                         ArgPart* arg, hipStream_t stream);

}  // namespace svhead
