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
// Design, per drafted position i (positions run in order, because x_i feeds
// position i + 1):
//   * The streaming path (rank r a multiple of 16 up to 256, V a multiple of
//     8: the heavy shape). One launch of mk_stream_kernel per position: every
//     CU streams 32-column vocabulary tiles for 256 requests while the
//     matrix cores form the bias A[x_{i-1}[b]] Bm^T in fp32 (rank r as the
//     depth); each bias is added to its backbone value, rounded once to bf16
//     and stored, so the bias never reaches memory. Each request's first
//     argmax over its stored row merges across the column slots through a
//     64-bit atomic maximum on an order-preserving key, and the next
//     position's launch decodes those keys into its rows of A. A seed launch
//     comes first and a last launch writes the final position's tokens:
//     K + 2 launches per call.
//   * Otherwise, two launches per position: the output head's product with
//     the previous tokens as its row map and an add-and-store epilogue (the
//     backbone values in and the drafter rows out with 16-byte accesses
//     through LDS), which also keeps a first argmax per row and vocabulary
//     split; then one wave per request merges its splits' entries (ties to
//     the lower column). The stored rows are not read back. 1 + 2K launches.
// The seed launch checks the given last tokens and writes the first row map.

#include <hip/hip_runtime.h>

#include <algorithm>
#include <climits>
#include <cmath>
#include <cstdint>

#include "head_gemm.h"
#include "lds_dma.h"
#include "spec_verify.h"

namespace {

using svhead::ArgPart;
using svhead::HeadRows;

constexpr int kMkPickThreads = 256;
constexpr int kMkPickWaves = kMkPickThreads / 64;     // one request per wave

constexpr int kMsGrid = 256;                       // streaming product: one workgroup per CU
constexpr int kMsRows = 256;                       // requests per workgroup

// Groups of 256 requests for B requests (a power of two up to 32): the
// streaming product's workgroups split into that many groups, each with
// kMsGrid / groups column slots.
inline int ms_halves(int B) {
    int nh = 1;
    while (nh * kMsRows < B) nh <<= 1;
    return nh;
}

struct MkLayout {
    size_t map0, map1, parts, keys, total;
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
    // First-argmax entries per request and vocabulary split of the
    // product path for other shapes.
    L.parts = take((size_t)svhead::add_splits(B, V) * (size_t)B * sizeof(ArgPart));
    // The streaming path's first-argmax keys: three arrays of B (position i
    // writes array i % 3, the next reads it, the one before clears i + 1's).
    L.keys = take((size_t)3 * B * sizeof(unsigned long long));
    L.total = o;
    return L;
}

// The first row map: the given last tokens; one outside [0, V) becomes -1 (a
// row of zeros in the product) and raises SV_FLAG_BAD_TOKEN.
// With `keys` (the streaming path) it also clears position 0's argmax keys.
__global__ void mk_seed_kernel(const int32_t* __restrict__ prev, int B, int V,
                               int32_t* __restrict__ map, int32_t* __restrict__ status,
                               unsigned long long* __restrict__ keys) {
    __shared__ int bad;
    if (threadIdx.x == 0) bad = 0;
    __syncthreads();
    int mine = 0;
    for (int b = threadIdx.x; b < B; b += blockDim.x) {
        const int t = prev[b];
        const bool ok = t >= 0 && t < V;
        map[b] = ok ? t : -1;
        mine |= ok ? 0 : 1;
        if (keys) keys[b] = 0ull;
    }
    if (mine) atomicOr(&bad, 1);
    __syncthreads();
    if (threadIdx.x == 0 && status) status[0] = bad ? (int32_t)SV_FLAG_BAD_TOKEN : 0;
}

__device__ __forceinline__ bool mk_better(float v, int i, float bv, int bi) {
    return v > bv || (v == bv && i < bi);
}

// A (value, column) entry as a 64-bit key whose unsigned order is
// mk_better's: the value's order-preserving bits (-0 taken as +0, so that
// equal values tie), then the column inverted, so an equal value at a lower
// column is larger. A column of INT_MAX (nothing taken) loses to every real
// column; the key 0 (no entry) decodes to no column. Values are never NaN.
__device__ __forceinline__ unsigned long long mk_key(float v, int i) {
    const unsigned u = __float_as_uint(v == 0.0f ? 0.0f : v);
    const unsigned hi = (u & 0x80000000u) ? ~u : (u | 0x80000000u);
    return ((unsigned long long)hi << 32) | (unsigned long long)(0xFFFFFFFFu - (unsigned)i);
}
// The drafted token of a merged key: its column, or 0 when no value above
// -inf was taken (the pick kernel's rule).
__device__ __forceinline__ int mk_key_token(unsigned long long key, int V) {
    const unsigned i = 0xFFFFFFFFu - (unsigned)key;
    return i < (unsigned)V ? (int)i : 0;
}

// The last position's tokens from its merged keys (the streaming path).
__global__ void mk_final_kernel(const unsigned long long* __restrict__ keys, int B, int K, int V,
                                int32_t* __restrict__ out_tokens) {
    const int b = blockIdx.x * blockDim.x + threadIdx.x;
    if (b < B) out_tokens[(size_t)b * K + K - 1] = mk_key_token(keys[b], V);
}


// ---------------------------------------------------------------------------
// The streaming product for rank r a multiple of 16 up to 256 and V a
// multiple of 8 (the bench's rank-256 shape). Per position the work is
// bound by HBM -- the backbone rows in, the drafter rows out, the factor Bm
// once -- so every CU streams vocabulary tiles of 32 columns for 256
// requests while the matrix cores form the bias:
//   * 8 waves, two per SIMD, so that one wave's LDS and memory waits pass
//     under the other's work; each keeps its 32 requests' rows of A
//     (x_{i-1}[b]'s row) as MFMA fragments in registers for the whole
//     launch (the transposed product: Bm's columns as the first operand, so
//     a lane holds one request's row and 16 columns of the 32 x 32 block);
//   * Bm's tile (32 rows of r) and the backbone's tiles (256 rows of 32
//     columns, taken in pairs so that each row moves as a 128-byte piece)
//     come in by buffer-to-LDS loads into a ring of 4 Bm slots (three tiles
//     ahead of use) and a ring of 3 pair slots (two pairs ahead); one wait
//     and one barrier per tile;
//   * tile t's bias is added to its backbone values, rounded once to bf16
//     and stored while tile t + 1's product runs, and the running maximum
//     of the stored values is kept per request, with the first tile that
//     reached it; the column within that tile is read back at the end.
// The workgroups that share a column slot (one per group of 256 requests)
// sit on one XCD and walk the same tiles, so the second one can find Bm's
// tiles in that XCD's L2 (about half of its loads do).
constexpr int kMsThreads = 512;                    // 8 waves, 32 requests each
constexpr int kMsCols = 32;                        // vocabulary columns per tile
constexpr int kMsMaxG = 16;                        // k-groups of 16: r <= 256
constexpr int kMsBmBytes = kMsCols * 512;          // one Bm tile: 32 rows of 512 bytes
constexpr int kMsPairBytes = kMsRows * kMsCols * 4;   // two backbone tiles: 256 rows of 128 bytes
constexpr int kMsBmSlots = 4;                      // Bm tiles three ahead
constexpr int kMsPairSlots = 3;                    // backbone pairs two ahead
constexpr int kMsLds = kMsBmSlots * kMsBmBytes + kMsPairSlots * kMsPairBytes;   // 160 KB
constexpr unsigned kMsOob = 0x80000000u;           // past every buffer's range

typedef __bf16 ms_bf16x8 __attribute__((ext_vector_type(8)));
typedef float ms_f32x16 __attribute__((ext_vector_type(16)));
typedef __bf16 ms_bf16x2 __attribute__((ext_vector_type(2)));
typedef float ms_f32x2 __attribute__((ext_vector_type(2)));
typedef unsigned ms_u32x4 __attribute__((ext_vector_type(4)));

// Two fp32 values to packed bf16 bits (lo in the low half), one
// v_cvt_pk_bf16_f32: to nearest, ties to even, under the default float
// mode; a NaN becomes the quiet NaN that keeps its sign and upper payload
// bits, i.e. the bits (u >> 16) | 0x40 of its pattern u.
__device__ __forceinline__ uint32_t ms_pack_bf16(float lo, float hi) {
    const ms_f32x2 v = {lo, hi};
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, ms_bf16x2));
}

// The LDS reads and writes of the epilogue, each waited for inside its asm
// block (read outputs are early-clobbered, so no result lands on an address
// still to be used). Written out because the compiler, seeing an LDS read
// while buffer-to-LDS loads into the same array are in flight, would
// otherwise wait for every one of those loads first, though the slot read
// has been ordered already.
__device__ __forceinline__ void ms_read4(uint2 (&v)[4], const unsigned (&ad)[4]) {
    asm volatile(
        "ds_read_b64 %0, %4\n\t"
        "ds_read_b64 %1, %5\n\t"
        "ds_read_b64 %2, %6\n\t"
        "ds_read_b64 %3, %7\n\t"
        "s_waitcnt lgkmcnt(0)"
        : "=&v"(v[0]), "=&v"(v[1]), "=&v"(v[2]), "=&v"(v[3])
        : "v"(ad[0]), "v"(ad[1]), "v"(ad[2]), "v"(ad[3])
        : "memory");
}
__device__ __forceinline__ void ms_write4(const uint2 (&v)[4], const unsigned (&ad)[4]) {
    asm volatile(
        "ds_write_b64 %0, %4\n\t"
        "ds_write_b64 %1, %5\n\t"
        "ds_write_b64 %2, %6\n\t"
        "ds_write_b64 %3, %7\n\t"
        "s_waitcnt lgkmcnt(0)"
        :
        : "v"(ad[0]), "v"(ad[1]), "v"(ad[2]), "v"(ad[3]), "v"(v[0]), "v"(v[1]), "v"(v[2]),
          "v"(v[3])
        : "memory");
}
__device__ __forceinline__ void ms_read4x16(uint4 (&v)[4], const unsigned (&ad)[4]) {
    asm volatile(
        "ds_read_b128 %0, %4\n\t"
        "ds_read_b128 %1, %5\n\t"
        "ds_read_b128 %2, %6\n\t"
        "ds_read_b128 %3, %7\n\t"
        "s_waitcnt lgkmcnt(0)"
        : "=&v"(v[0]), "=&v"(v[1]), "=&v"(v[2]), "=&v"(v[3])
        : "v"(ad[0]), "v"(ad[1]), "v"(ad[2]), "v"(ad[3])
        : "memory");
}
__device__ __forceinline__ void ms_read2x16(uint4 (&v)[2], const unsigned (&ad)[2]) {
    asm volatile(
        "ds_read_b128 %0, %2\n\t"
        "ds_read_b128 %1, %3\n\t"
        "s_waitcnt lgkmcnt(0)"
        : "=&v"(v[0]), "=&v"(v[1])
        : "v"(ad[0]), "v"(ad[1])
        : "memory");
}

// The LDS byte address of p (a pointer into dynamic shared memory).
__device__ __forceinline__ unsigned ms_lds_addr(const void* p) {
    return (unsigned)(uintptr_t)(const __attribute__((address_space(3))) void*)p;
}

// The streaming path's condition.
inline bool ms_path(int B, int K, int V, int r) {
    return r % 16 == 0 && r <= 16 * kMsMaxG && V % 8 == 0 && B <= 32 * kMsRows &&
           (unsigned long long)B * K * V * 2 <= kMsOob && (unsigned long long)V * r * 2 <= kMsOob;
}

__global__ __launch_bounds__(kMsThreads) __attribute__((amdgpu_waves_per_eu(2, 2)))
void mk_stream_kernel(const uint16_t* __restrict__ A, const uint16_t* __restrict__ Bm,
                      const int32_t* __restrict__ map, const unsigned long long* __restrict__ kin,
                      unsigned long long* __restrict__ kout, unsigned long long* __restrict__ kclear,
                      const uint16_t* __restrict__ base, uint16_t* __restrict__ out, int B, int K,
                      int V, int r, int pos, int nh, int32_t* __restrict__ out_tokens) {
    extern __shared__ __align__(16) unsigned char ms_lds[];
    unsigned char* const bm_lds = ms_lds;
    unsigned char* const base_lds = ms_lds + kMsBmSlots * kMsBmBytes;
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane((int)threadIdx.x >> 6);
    const int xcd = (int)blockIdx.x % 8, idx = (int)blockIdx.x / 8;
    const int half = idx % nh;
    const int S = kMsGrid / nh;                    // column slots
    const int slot = xcd * (32 / nh) + idx / nh;
    const int row0 = half * kMsRows;
    if (row0 >= B) return;                         // no requests here (whole workgroup)
    const int ntile = (V + kMsCols - 1) / kMsCols;
    const int ng = r / 16;
    // The slot's tiles are a contiguous range t0 .. t0 + nj - 1 of the row,
    // whole pairs of tiles (t0 even) but for the row's last, so that two
    // tiles' rows leave as 128-byte segments.
    const int npair = (ntile + 1) / 2;
    const int t0 = 2 * (int)((long long)slot * npair / S);
    const int nj = std::min(2 * (int)((long long)(slot + 1) * npair / S), ntile) - t0;
    const long long rowlen = (long long)K * V;     // elements between one request's rows

    // This lane's request: tile row trow = 32 wave + l % 32, request
    // row0 + trow (lanes l and l + 32 share it, k-pieces l / 32).
    const int trow = wave * 32 + (lane & 31);
    const int req = row0 + trow;
    ms_bf16x8 af[kMsMaxG];
    {
        // The previous token: the given one (map, -1 when invalid) at
        // position 0, else the merged key of position pos - 1, whose token
        // the column slot 0 workgroups write out. Those also clear position
        // pos + 1's keys (read by no launch until then).
        int x = -1;
        if (req < B) {
            if (kin == nullptr) {
                x = map[req];
            } else {
                x = mk_key_token(kin[req], V);
                if (slot == 0 && lane < 32) out_tokens[(size_t)req * K + pos - 1] = x;
            }
            if (slot == 0 && lane < 32) kclear[req] = 0ull;
        }
        const uint16_t* arow = A + (size_t)(x < 0 ? 0 : x) * r + 8 * (lane >> 5);
        #pragma unroll
        for (int g = 0; g < kMsMaxG; ++g) {
            ms_bf16x8 v = {};
            if (g < ng && x >= 0) v = *reinterpret_cast<const ms_bf16x8*>(arow + 16 * g);
            af[g] = v;
        }
    }

    const __amdgpu_buffer_rsrc_t bm_rs = svdma::rsrc(Bm, (unsigned)((size_t)V * r * 2));
    // The backbone's and the stored rows' range ends with request B - 1's
    // row of this position.
    const unsigned row_range = (unsigned)(((size_t)(B - 1) * rowlen + V) * 2);
    const __amdgpu_buffer_rsrc_t base_rs = svdma::rsrc(base, row_range);
    const __amdgpu_buffer_rsrc_t out_rs = svdma::rsrc(out, row_range);

    // Loads. Bm, tile j, 2 per wave: instruction q = 2 wave + n moves rows
    // 2q, 2q + 1 of the tile, lane l row 2q + l / 32, its 16-byte piece
    // l % 32 holding k-piece (l % 32) ^ (row % 16) (pieces past r / 8 and
    // rows past V read zeros). Backbone, tiles 2P and 2P + 1 as one pair of
    // 128-byte row segments, 4 per wave: instruction q = 4 wave + n moves
    // rows 8q .. 8q + 7, lane l row 8q + l / 8 at position l % 8, which holds
    // the row's 16-byte piece (l % 8) ^ (row % 8), columns 8 of them from
    // the pair's first (requests past B read zeros): a wave moves its own
    // requests' rows. The lane parts of the offsets are fixed; a tile or a
    // pair adds its first column's (an offset past the range stays past it).
    unsigned bm_off[2], bp_off[4];
    #pragma unroll
    for (int n = 0; n < 2; ++n) {
        const int q = 2 * wave + n;
        const int row = 2 * q + (lane >> 5);
        const int p = (lane & 31) ^ (row & 15);
        bm_off[n] = p < r / 8 ? (unsigned)row * (unsigned)(2 * r) + 16u * (unsigned)p : kMsOob;
    }
    #pragma unroll
    for (int n = 0; n < 4; ++n) {
        const int row = 8 * (4 * wave + n) + (lane >> 3);
        const int b = row0 + row;
        bp_off[n] = b < B ? (unsigned)((long long)b * rowlen * 2) +
                                16u * (unsigned)((lane & 7) ^ (row & 7))
                          : kMsOob;
    }
    auto issue_bm = [&](int j) {
        const unsigned v0 = (unsigned)((t0 + j) * kMsCols);
        unsigned char* dst = bm_lds + (j % kMsBmSlots) * kMsBmBytes;
        #pragma unroll
        for (int n = 0; n < 2; ++n)
            svdma::load16(bm_rs, bm_off[n] + v0 * (unsigned)(2 * r), dst + (2 * wave + n) * 1024);
    };
    // The backbone is read once and the stored rows are not read again, so
    // both go non-temporal: they leave the L2 first and Bm's tiles, which the
    // slot's other workgroup reads too, stay.
    auto issue_pair = [&](int P) {
        const unsigned vp = (unsigned)((t0 + 2 * P) * kMsCols);
        unsigned char* dst = base_lds + (P % kMsPairSlots) * kMsPairBytes;
        #pragma unroll
        for (int n = 0; n < 4; ++n)
            svdma::load16<2>(base_rs, bp_off[n] + 2u * vp, dst + (4 * wave + n) * 1024);
    };

    // The running maximum of this lane's stored values over its columns,
    // and the first tile that reached it (-1: none yet).
    float bv = -INFINITY;
    int bt = -1;
    ms_f32x16 acc[2];                              // [tile parity]

    // Tile j's bias into c: Bm's fragment of k-group g is lane l's row
    // l % 32, k-piece 2 g + l / 32. Every k-group takes part: past r / 8
    // pieces both operands hold zeros.
    auto product = [&](int j, ms_f32x16& c) {
        const unsigned char* src = bm_lds + (j % kMsBmSlots) * kMsBmBytes + (lane & 31) * 512;
        ms_bf16x8 bf[kMsMaxG];
        #pragma unroll
        for (int g = 0; g < kMsMaxG; ++g)
            bf[g] = *reinterpret_cast<const ms_bf16x8*>(src + 16 * ((2 * g + (lane >> 5)) ^ (lane & 15)));
        const ms_f32x16 zero = {};
        c = __builtin_amdgcn_mfma_f32_32x32x16_bf16(bf[0], af[0], zero, 0, 0, 0);
        #pragma unroll
        for (int g = 1; g < kMsMaxG; ++g)
            c = __builtin_amdgcn_mfma_f32_32x32x16_bf16(bf[g], af[g], c, 0, 0, 0);
    };

    // The epilogue's lane parts, within a pair's slot: the backbone values
    // of row trow, columns 4 (l / 32) + 8 q .. + 4 of the pair's first tile,
    // sit at ad0[q] (of its second tile at ad0[q] ^ 64: piece q + 4); the
    // store pieces of a pair (row 8 (4 wave + n) + l / 8, columns
    // 8 (l % 8) .. + 8 of the pair) at pa0[n], their rows at pr_off[n]; those
    // of a lone first tile (row 16 (2 wave + n) + l / 4, columns
    // 8 (l % 4) .. + 8) at sa0[n], their rows at st_off[n] (offsets past the
    // range for requests past B).
    unsigned ad0[4], pa0[4], pr_off[4], sa0[2], st_off[2];
    #pragma unroll
    for (int q = 0; q < 4; ++q)
        ad0[q] = (unsigned)(trow * 128 + 16 * (q ^ (trow & 7)) + 8 * (lane >> 5));
    #pragma unroll
    for (int n = 0; n < 4; ++n) {
        const int row = 8 * (4 * wave + n) + (lane >> 3);
        pa0[n] = (unsigned)(row * 128 + 16 * ((lane & 7) ^ (row & 7)));
        pr_off[n] = row0 + row < B ? (unsigned)((long long)(row0 + row) * rowlen * 2) +
                                         16u * (unsigned)(lane & 7)
                                   : kMsOob;
    }
    #pragma unroll
    for (int n = 0; n < 2; ++n) {
        const int row = 16 * (2 * wave + n) + (lane >> 2);
        sa0[n] = (unsigned)(row * 128 + 16 * ((lane & 3) ^ (row & 7)));
        st_off[n] = row0 + row < B ? (unsigned)((long long)(row0 + row) * rowlen * 2) +
                                         16u * (unsigned)(lane & 3)
                                   : kMsOob;
    }

    // Tile j's rows out: lane l's values are columns v0 + 4 (l / 32) + 8 q
    // + e (q, e < 4), element 4 q + e of the block. The rounded values go
    // back into the pair's slot (each lane where it read its backbone
    // values) and leave from there once the pair is complete, as 16-byte
    // pieces, 8 lanes a 128-byte row segment. A wave's backbone rows are its
    // own in both layouts, so the slot needs no barrier.
    // `out_mode`: 0 keeps tile j (even) in its pair's slot, 1 stores the
    // pair with tile j (odd), 2 stores tile j alone (the row's last tile,
    // even and unpaired).
    auto finish = [&](int j, const ms_f32x16& c, int out_mode) {
        const int v0 = (t0 + j) * kMsCols;
        const unsigned sb = ms_lds_addr(base_lds + ((j >> 1) % kMsPairSlots) * kMsPairBytes);
        const unsigned hx = out_mode == 1 ? 64u : 0u;   // the pair's second tile
        unsigned ad[4];
        #pragma unroll
        for (int q = 0; q < 4; ++q) ad[q] = sb + (ad0[q] ^ hx);
        uint2 bw[4];
        ms_read4(bw, ad);
        float sm[16];
        #pragma unroll
        for (int q = 0; q < 4; ++q) {
            sm[4 * q] = __uint_as_float(bw[q].x << 16) + c[4 * q];
            sm[4 * q + 1] = __uint_as_float(bw[q].x & 0xFFFF0000u) + c[4 * q + 1];
            sm[4 * q + 2] = __uint_as_float(bw[q].y << 16) + c[4 * q + 2];
            sm[4 * q + 3] = __uint_as_float(bw[q].y & 0xFFFF0000u) + c[4 * q + 3];
            bw[q] = make_uint2(ms_pack_bf16(sm[4 * q], sm[4 * q + 1]),
                               ms_pack_bf16(sm[4 * q + 2], sm[4 * q + 3]));
        }
        ms_write4(bw, ad);
        if (out_mode == 1) {
            const int vp = v0 - kMsCols;           // the pair's first column
            unsigned sa[4];
            #pragma unroll
            for (int n = 0; n < 4; ++n) sa[n] = sb + pa0[n];
            uint4 ov[4];
            ms_read4x16(ov, sa);
            #pragma unroll
            for (int n = 0; n < 4; ++n) {
                const unsigned off =
                    vp + 8 * (lane & 7) < V ? pr_off[n] + 2u * (unsigned)vp : kMsOob;
                const ms_u32x4 d = {ov[n].x, ov[n].y, ov[n].z, ov[n].w};
                __builtin_amdgcn_raw_buffer_store_b128(d, out_rs, off, 0, 2);
            }
        } else if (out_mode == 2) {
            unsigned sa[2];
            #pragma unroll
            for (int n = 0; n < 2; ++n) sa[n] = sb + sa0[n];
            uint4 ov[2];
            ms_read2x16(ov, sa);
            #pragma unroll
            for (int n = 0; n < 2; ++n) {
                const unsigned off =
                    v0 + 8 * (lane & 3) < V ? st_off[n] + 2u * (unsigned)v0 : kMsOob;
                const ms_u32x4 d = {ov[n].x, ov[n].y, ov[n].z, ov[n].w};
                __builtin_amdgcn_raw_buffer_store_b128(d, out_rs, off, 0, 2);
            }
        }
        // Columns from V on (only in the row's last tile) take no part.
        if (v0 + kMsCols > V) {
            const int c0 = v0 + 4 * (lane >> 5);
            #pragma unroll
            for (int k = 0; k < 16; ++k)
                sm[k] = c0 + 8 * (k >> 2) + (k & 3) < V ? sm[k] : __uint_as_float(0x7FC00000u);
        }
        // The sums' maximum (fmaxf drops NaNs) rounds to the maximum of the
        // stored values, rounding being monotone. A lane meets its columns in
        // increasing order, over the elements and the tiles, so the first
        // tile that reaches the maximum holds the first argmax, unless no
        // tile has been taken yet (an equal value, -inf, wins only then).
        float m[8];
        #pragma unroll
        for (int k = 0; k < 8; ++k) m[k] = fmaxf(sm[k], sm[k + 8]);
        #pragma unroll
        for (int k = 0; k < 4; ++k) m[k] = fmaxf(m[k], m[k + 4]);
        const float ms = fmaxf(fmaxf(m[0], m[2]), fmaxf(m[1], m[3]));
        const float mx = __uint_as_float(ms_pack_bf16(ms, ms) << 16);
        const bool take = (mx > bv) | ((mx == bv) & (bt < 0));
        bv = take ? mx : bv;
        bt = take ? j : bt;
    };

    // Load order, as if steps -4 .. -1 had run: step s issues backbone pair
    // s / 2 + 2 when s is even, then Bm tile s + 3, so pair 0 and Bm tiles
    // 0 .. 2 and pair 1 go out first; every step issues its loads, past the
    // last tile too (into slots that are not read again), so each wait
    // counts the same loads. Step j waits for Bm tile j (and every earlier
    // load: pair (j - 1) / 2 went out before it); after it come Bm tiles
    // j + 1 and j + 2 (2 loads each) and one pair (4). It passes the barrier
    // that makes the Bm tile visible and frees tile j - 1's Bm slot,
    // finishes tile j - 1 (storing the pair when j - 1 is odd, which frees
    // that pair's slot for the pair issued next), issues and forms tile j's
    // bias; the loop is unrolled by two so that each half takes one
    // accumulator parity and one tile parity.
    if (nj > 0) {
        issue_pair(0);
        issue_bm(0);
        issue_pair(1);
        issue_bm(1);
        issue_bm(2);
        svdma::wait_vm<8>();
        svdma::ring_barrier();
        issue_pair(2);
        issue_bm(3);
        product(0, acc[0]);
        auto step = [&](int j, ms_f32x16& cur, const ms_f32x16& prev, int out_mode) {
            svdma::wait_vm<8>();
            svdma::ring_barrier();
            finish(j - 1, prev, out_mode);
            if (out_mode == 1) issue_pair(j / 2 + 2);
            issue_bm(j + 3);
            product(j, cur);
        };
        for (int j = 1; j < nj; j += 2) {
            step(j, acc[1], acc[0], 0);            // tile j - 1 even: kept
            if (j + 1 < nj) step(j + 1, acc[0], acc[1], 1);   // tile j odd: the pair leaves
        }
        // The last pair's backbone went out at least 16 loads before the end.
        svdma::wait_vm<16>();
        if (nj & 1) finish(nj - 1, acc[0], 2);
        else finish(nj - 1, acc[1], 1);
    }

    // The lane's first column holding its maximum, in the tile that first
    // reached it: that tile's stored values of the request, read back once
    // the wave's stores are complete (the wave stored them itself; the loads
    // bypass the vector L1). Columns from V on are not read, and a valid
    // column reaches the maximum before them.
    svdma::wait_vm<0>();
    int bi = INT_MAX;
    if (bt >= 0) {
        const int c0 = (t0 + bt) * kMsCols + 4 * (lane >> 5);
        uint2 w[4];
        #pragma unroll
        for (int q = 0; q < 4; ++q) {
            const int col = c0 + 8 * q;
            const unsigned off = col < V ? (unsigned)(((long long)req * rowlen + col) * 2) : kMsOob;
            w[q] = __builtin_bit_cast(uint2, __builtin_amdgcn_raw_buffer_load_b64(out_rs, off, 0, 1));
        }
        #pragma unroll
        for (int k = 15; k >= 0; --k) {
            const uint32_t h = (k & 2) ? w[k >> 2].y : w[k >> 2].x;
            const float v = __uint_as_float((k & 1) ? (h & 0xFFFF0000u) : (h << 16));
            bi = v == bv ? c0 + 8 * (k >> 2) + (k & 3) : bi;
        }
    }

    // The lane pair holding a request merges, lane < 32 writes its partial.
    {
        const float ov = __shfl_xor(bv, 32, 64);
        const int oi = __shfl_xor(bi, 32, 64);
        if (mk_better(ov, oi, bv, bi)) {
            bv = ov;
            bi = oi;
        }
        // Merged over the column slots by an atomic maximum of the keys.
        if (lane < 32 && req < B) atomicMax(kout + req, mk_key(bv, bi));
    }
    svdma::wait_vm<0>();                           // the last stores
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

    const bool streamed = ms_path(B, K, V, r);
    unsigned long long* keys = reinterpret_cast<unsigned long long*>(ws + L.keys);
    hipLaunchKernelGGL(mk_seed_kernel, dim3(1), dim3(1024), 0, s, prev_tokens, B, V, map[0],
                       out_status, streamed ? keys : nullptr);
    if (hipGetLastError() != hipSuccess) return SV_ERR_HIP;
    if (streamed) {
        static const hipError_t attr = hipFuncSetAttribute(
            reinterpret_cast<const void*>(&mk_stream_kernel),
            hipFuncAttributeMaxDynamicSharedMemorySize, kMsLds);
        if (attr != hipSuccess) return SV_ERR_HIP;
        // One launch per position: position i merges its first argmaxes
        // into keys array i % 3, reads position i - 1's and clears i + 1's;
        // a last small launch writes position K - 1's tokens.
        const int nh = ms_halves(B);
        auto kbuf = [&](int i) { return keys + (size_t)(i % 3) * B; };
        for (int i = 0; i < K; ++i) {
            hipLaunchKernelGGL(mk_stream_kernel, dim3(kMsGrid), dim3(kMsThreads), kMsLds, s, A, Bm,
                               map[0], i > 0 ? kbuf(i - 1) : nullptr, kbuf(i), kbuf(i + 1),
                               base + (size_t)i * V, out + (size_t)i * V, B, K, V, r, i, nh,
                               out_tokens);
            if (hipGetLastError() != hipSuccess) return SV_ERR_HIP;
        }
        hipLaunchKernelGGL(mk_final_kernel, dim3((unsigned)((B + 255) / 256)), dim3(256), 0, s,
                           kbuf(K - 1), B, K, V, out_tokens);
        if (hipGetLastError() != hipSuccess) return SV_ERR_HIP;
        return SV_OK;
    }
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
