// sa_internal.h -- launchers behind the C ABI (no validation here: the
// entry points in sa_api.cpp check shapes and pointers first).
#pragma once
#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace sa {

struct Shape {
    int batch, T, heads, kv_heads, causal;
    const int32_t* seqlens;  // device pointer or nullptr
    int block_order;
    int v_rows;  // 1: V and dV as rows [T][64] (like K), 0: V^T and dV^T
};

// Block schedules of the kernels whose blocks take query tiles (forward,
// query pass, dQ pass).  Pairs: each block takes the tiles (n - 1 - p, p),
// whose causal walks add up to the same length, so a grid of many rounds
// drains evenly; single: one tile per block, the longest first, used when a
// grid of single tiles fits the chip at once (two blocks on each of 256 CUs),
// where pairing would only halve the blocks in flight; plain: one tile per
// block in natural order (the caller's block_order = 1).  Every schedule
// gives bitwise the same results.
constexpr int kOrderPairs = 0, kOrderPlain = 1, kOrderSingle = 2;
// The key pass's own pairing: one workgroup takes key tiles p and nkt - 1 - p
// of a (batch, K/V head) one after the other (causal walks that add up to the
// same length), used when that grid fits the chip in one round.
constexpr int kOrderKeyPairs = 3;
constexpr size_t kChipCUs = 256;  // MI355X: 8 XCDs of 32 CUs
constexpr size_t kSingleTileGridMax = 2 * kChipCUs;
inline int tile_schedule(const Shape& sh, size_t units, int n_tiles) {
    if (sh.block_order == 1) return kOrderPlain;
    return units * (size_t)n_tiles <= kSingleTileGridMax ? kOrderSingle : kOrderPairs;
}
inline size_t tile_schedule_blocks(int order, size_t units, int n_tiles) {
    return units * (order == kOrderPairs ? (size_t)(n_tiles + 1) / 2 : (size_t)n_tiles);
}

// dS workspace geometry: one fp16 64x64 tile per (batch, query head, query
// tile qt, key tile kt) that the dQ pass reads.  Causal: kt <= qt, tile index
// qt (qt + 1) / 2 + kt; otherwise the full square, qt * nt + kt.
inline size_t ds_tiles_per_head(const Shape& sh) {
    size_t nt = (size_t)sh.T / 64;
    return sh.causal ? nt * (nt + 1) / 2 : nt * nt;
}
constexpr size_t kDsTileBytes = 64 * 64 * 2;
// Per-head index of the first dS tile of query tile row q (rows below q hold
// this many tiles).
inline long long ds_row_start(const Shape& sh, int q) {
    const long long nt = sh.T / 64;
    return sh.causal ? (long long)q * (q + 1) / 2 : (long long)q * nt;
}

// A query-row chunk of the split backward: the 64-row query tiles
// [q_lo, q_hi) (q_lo even, so that the dQ pass's 128-row blocks do not
// straddle chunks).  Their dS tiles sit in the workspace at per-head index
// (tile index - tile0), tph tiles per head.  accumulate: the key pass adds its
// dK and dV to what the outputs already hold (every chunk after the first).
struct Chunk {
    int q_lo, q_hi;
    long long tile0, tph;
    int accumulate;
};
inline Chunk whole_problem(const Shape& sh) {
    return Chunk{0, sh.T / 64, 0, (long long)ds_tiles_per_head(sh), 0};
}
// dS bytes a chunk needs.
inline size_t chunk_bytes(const Shape& sh, int q_lo, int q_hi) {
    return (size_t)sh.batch * sh.heads * (size_t)(ds_row_start(sh, q_hi) - ds_row_start(sh, q_lo)) * kDsTileBytes;
}
// The largest single 128-row block's dS: the least workspace a chunked
// backward can run in.
inline size_t largest_block_bytes(const Shape& sh) {
    const int nt = sh.T / 64;
    size_t most = 0;
    for (int q = 0; q < nt; q += 2) {
        const size_t b = chunk_bytes(sh, q, q + 2 < nt ? q + 2 : nt);
        if (b > most) most = b;
    }
    return most;
}
// The next chunk below query tile q_hi (> 0): as many 128-row blocks,
// downwards from q_hi, as fit in ws_bytes (at least one; the caller checks
// ws_bytes >= largest_block_bytes).  Chunks taken from the last rows to the
// first: the first one reaches every key tile, every later one accumulates.
inline Chunk next_chunk(const Shape& sh, int q_hi, size_t ws_bytes, bool first) {
    int q_lo = ((q_hi - 1) / 2) * 2;
    while (q_lo >= 2 && chunk_bytes(sh, q_lo - 2, q_hi) <= ws_bytes) q_lo -= 2;
    return Chunk{q_lo, q_hi, ds_row_start(sh, q_lo), ds_row_start(sh, q_hi) - ds_row_start(sh, q_lo),
                 first ? 0 : 1};
}

hipError_t launch_forward(const Shape& sh, const void* Q, const void* K, const void* Vt, void* O, float* L,
                          float c, hipStream_t stream);
hipError_t launch_row_terms(const Shape& sh, const void* dO, const void* O, float* D, hipStream_t stream);
hipError_t launch_key_pass(const Shape& sh, const void* Q, const void* K, const void* Vt, const void* dO,
                           const float* L, const float* D, void* dS, float c, float s, float* dK, float* dVt,
                           hipStream_t stream);
hipError_t launch_dq_pass(const Shape& sh, const void* K, const void* dS, float s, float* dQ,
                          hipStream_t stream);
// The split backward's key and dQ passes in query-row chunks over a dS
// workspace of ws_bytes (which may be far smaller than the whole problem's):
// chunks from the last rows to the first, each its key pass (dK and dV
// accumulated across chunks in that fixed order) then its dQ pass.  The row
// terms are not included.  Returns hipErrorInvalidValue, before launching
// anything, if a single 128-row chunk does not fit.
hipError_t launch_key_dq_chunked(const Shape& sh, const void* Q, const void* K, const void* Vt, const void* dO,
                                 const float* L, const float* D, void* ws, size_t ws_bytes, float c, float s,
                                 float* dQ, float* dK, float* dVt, hipStream_t stream);
// The smallest workspace launch_key_dq_chunked accepts for the shape.
size_t min_chunk_bytes(const Shape& sh);
// The dQ pass with the rotated epilogue: dQ turned back by the inverse
// half-split rotation (tables cos_t, sin_t fp32 [T][32]) and stored as the
// bfloat16 Q slice of the token-major projection gradient dqkv [B][T][width].
struct DqEpilogue {
    const float* cos;
    const float* sin;
    uint16_t* out;    // bfloat16 output (rotated slice, or the projection's bfloat16 copy)
    float* out32;     // the projection's binary32 copy
    int width;
};
hipError_t launch_dq_pass_rotated(const Shape& sh, const void* K, const void* dS, float s, const float* cos_t,
                                  const float* sin_t, void* dqkv, int width, hipStream_t stream);
// One column slice of a fused projection's token-major gradient [B][T][width]:
// head u's 64 values of row p at f32 / b16 + (b T + p) width + 64 u + d.
struct ProjectionOut {
    float* f32;
    uint16_t* b16;
    int width;
};
hipError_t launch_key_pass_projection(const Shape& sh, const void* Q, const void* K, const void* Vt,
                                      const void* dO, const float* L, const float* D, void* dS, float c, float s,
                                      const ProjectionOut& kproj, const ProjectionOut& vproj, hipStream_t stream);
hipError_t launch_dq_pass_projection(const Shape& sh, const void* K, const void* dS, float s, const ProjectionOut& q,
                                     hipStream_t stream);
hipError_t launch_query_pass_projection(const Shape& sh, const void* dO, const void* O, const float* L,
                                        const void* Q, const void* K, const void* Vt, float c, float s, float* D,
                                        const ProjectionOut& qproj, hipStream_t stream);
// The two-launch backward's query pass (D and dQ); its key launch is
// launch_key_pass with dS == nullptr (no score gradients stored).
hipError_t launch_query_pass(const Shape& sh, const void* dO, const void* O, const float* L, const void* Q,
                             const void* K, const void* Vt, float c, float s, float* D, float* dQ,
                             hipStream_t stream);

// Grid sizes, for the entry points' admission of launch dimensions.
size_t forward_blocks(const Shape& sh);
size_t row_terms_blocks(const Shape& sh);
size_t key_pass_blocks(const Shape& sh);
size_t dq_pass_blocks(const Shape& sh);
size_t query_pass_blocks(const Shape& sh);

}  // namespace sa
