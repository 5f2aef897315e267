// head_gemm.h -- internal interface of the output-head matrix product
// (head_stats.hip) for the other translation units of the library. Not part
// of the C ABI.
//
// The product z = h W^T of bf16 hidden states and the shared head runs on the
// matrix cores with one of four epilogues: per-row statistics for sampled or
// greedy verification, the fp32 logits themselves for a few rows, or the
// logits added to bf16 rows and stored rounded (the Markov head's transition
// term on the backbone's logits). Every epilogue accumulates each logit in
// the same order, so the logits written for a row equal, bit for bit, the
// values its statistics were taken over.
#pragma once

#include <hip/hip_runtime.h>

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
