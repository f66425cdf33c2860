// sa_forward.hip -- the streaming forward pass on gfx950.
//
// Method: StreamingAttentionSM86 page, banner "Causal attention as a
// streaming normalised sum".  For each 64-key tile up to the diagonal, a
// query row's scores are folded into a running maximum m, a running sum l and
// a running weighted sum O; a new maximum m' rescales l and O by 2^(m - m').
// Scores are base-2 (t = S c), P = 2^(t - m') is rounded to binary16 before
// P V, every sum is binary32, and the pass writes O / l and L = m + log2 l.
// Length masks and zero rows follow the variable-length gist page.
//
// MI355X design (not the pages' SM86 one): a 256-thread workgroup (4 wave64s)
// takes 128 queries of one query head; each wave owns 32 queries.  Each key
// tile's K rows and V^T rows are staged once in LDS for all four waves with
// coalesced 16-byte loads, double-buffered, the next tile's global loads in
// flight while the current tile computes.  A wave computes S^T = K Q^T with
// v_mfma_f32_32x32x16_f16 (A = K rows from LDS, B = the wave's Q kept in
// registers), so every lane holds 32 scores of ONE query: the row maximum is
// an in-lane max plus one v_permlane32_swap, the row sum stays a per-lane
// partial until the end (as the pages keep it per thread), and the rescale
// factor is per lane.  The fp16 P^T accumulators feed O^T += V^T P^T directly
// as the B operand: the contraction order over the tile's keys is permuted to
// match the accumulator layout, and V^T's A operand is read from LDS in the
// same permuted order, so P never leaves registers.
#include "sa_device.h"
#include "sa_internal.h"

namespace sa {

namespace {

constexpr int kFwdWaves = 4;
constexpr int kFwdRows = 32 * kFwdWaves;     // queries per workgroup
constexpr int kFwdThreads = 64 * kFwdWaves;
constexpr int kTileHalves = kTile * kLdsRow; // one padded 64-row tile in LDS

template <bool CAUSAL, bool VARLEN>
__global__ __launch_bounds__(kFwdThreads, 2) void sa_forward_kernel(
    const half_t* __restrict__ Q, const half_t* __restrict__ K, const half_t* __restrict__ Vt,
    half_t* __restrict__ O, float* __restrict__ L, const int32_t* __restrict__ seqlens, float c, int T,
    int H, int KV, int n_qtiles, int BH, int block_order) {
    __shared__ __attribute__((aligned(16))) half_t lds[2][2][kTileHalves];  // [buffer][K | V^T][row][col]

    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
    const int l32 = lane & 31, hi = lane >> 5;

    // Block -> (query tile, batch*head).  Order 0 walks the query tiles from
    // the last (longest causal walk) down, one tile of every head at a time.
    int qtile, bh;
    if (block_order == 0) {
        qtile = n_qtiles - 1 - (int)(blockIdx.x / BH);
        bh = (int)(blockIdx.x % BH);
    } else {
        qtile = (int)(blockIdx.x % n_qtiles);
        bh = (int)(blockIdx.x / n_qtiles);
    }
    const int b = bh / H, h = bh % H, kv = h / (H / KV);
    const int len = VARLEN ? min(max(seqlens[b], 0), T) : T;
    const int q0 = qtile * kFwdRows;
    const int qw = q0 + 32 * wave;                 // this wave's first query
    const int q = qw + l32;                        // this lane's query
    const bool wave_rows = qw < T;                 // T % 64 == 0: whole wave in or out
    const int row_limit = VARLEN ? len : T;        // rows at or past it are masked

    // Key tiles the block walks, and the keys each wave needs.
    int kend = CAUSAL ? min(q0 + kFwdRows, T) : T;
    if (VARLEN) kend = min(kend, len);
    const int n_kt = (kend + kTile - 1) / kTile;
    int kend_w = CAUSAL ? qw + 32 : T;
    if (VARLEN) kend_w = min(kend_w, len);
    const bool wave_live = wave_rows && qw < row_limit;

    const size_t kv_off = ((size_t)b * KV + kv) * (size_t)T * kHeadDim;
    const half_t* Kp = K + kv_off;
    const half_t* Vp = Vt + kv_off;

    // Q^T as the B operand of S^T = K Q^T: lane (query l32, half hi) holds
    // Q[q][16 s + 8 hi + 0..7] for s = 0..3.
    half8 qf[4];
    if (wave_live) {
        const half_t* qp = Q + (((size_t)b * H + h) * T + q) * kHeadDim + 8 * hi;
#pragma unroll
        for (int s = 0; s < 4; ++s) qf[s] = *(const half8*)(qp + 16 * s);
    }

    f32x16 oacc[2] = {zero16(), zero16()};  // O^T, d blocks 0..31 and 32..63
    float m = kNegInf, lsum = 0.0f;

    // Staging: 512 16-byte chunks per 64x64 tile; thread tid moves chunks
    // tid and tid + 256 of K and of V^T.
    uint4 kreg[2], vreg[2];
    auto load_tile = [&](int j) {
#pragma unroll
        for (int u = 0; u < 2; ++u) {
            int chunk = tid + u * kFwdThreads, row = chunk >> 3, col = (chunk & 7) * 8;
            kreg[u] = *(const uint4*)(Kp + (size_t)(j * kTile + row) * kHeadDim + col);
            vreg[u] = *(const uint4*)(Vp + (size_t)row * T + j * kTile + col);
        }
    };
    auto store_tile = [&](int j, int buf) {
#pragma unroll
        for (int u = 0; u < 2; ++u) {
            int chunk = tid + u * kFwdThreads, row = chunk >> 3, col = (chunk & 7) * 8;
            uint4 v = vreg[u];
            if (VARLEN && j * kTile + col + 8 > len) {
                // Keys at or past the length contribute P = 0; clear their V
                // entries so that no padding value can reach O.
                half_t* e = (half_t*)&v;
#pragma unroll
                for (int t = 0; t < 8; ++t)
                    if (j * kTile + col + t >= len) e[t] = (half_t)0.0f;
            }
            *(uint4*)&lds[buf][0][row * kLdsRow + col] = kreg[u];
            *(uint4*)&lds[buf][1][row * kLdsRow + col] = v;
        }
    };

    if (n_kt > 0) {
        load_tile(0);
        store_tile(0, 0);
    }
    __syncthreads();

    for (int j = 0; j < n_kt; ++j) {
        const int buf = j & 1;
        if (j + 1 < n_kt) load_tile(j + 1);

        if (wave_live && j * kTile < kend_w) {
            const half_t* Ks = lds[buf][0];
            const half_t* Vs = lds[buf][1];
            // S^T = K Q^T for the tile's two 32-key blocks.
            f32x16 sacc[2] = {zero16(), zero16()};
#pragma unroll
            for (int s = 0; s < 4; ++s) {
#pragma unroll
                for (int kb = 0; kb < 2; ++kb) {
                    half8 a = *(const half8*)(Ks + (32 * kb + l32) * kLdsRow + 16 * s + 8 * hi);
                    sacc[kb] = mfma32(a, qf[s], sacc[kb]);
                }
            }
            // Mask: key past the query (causal) or at/past the length.  Only
            // tiles that reach past the wave's first query or the length.
            const int key0 = j * kTile;
            const bool need_mask = (CAUSAL && key0 + kTile - 1 > qw) ||
                                   (VARLEN && (key0 + kTile > len || qw + 32 > len));
            if (need_mask) {
#pragma unroll
                for (int kb = 0; kb < 2; ++kb)
#pragma unroll
                    for (int r = 0; r < 16; ++r) {
                        int key = key0 + 32 * kb + 8 * (r >> 2) + 4 * hi + (r & 3);
                        bool masked = (CAUSAL && key > q) || (VARLEN && (key >= len || q >= len));
                        sacc[kb][r] = masked ? kNegInf : sacc[kb][r];
                    }
            }
            // Row maximum of the raw scores (c > 0, so max(S) c = max(S c)).
            float mx = sacc[0][0];
#pragma unroll
            for (int kb = 0; kb < 2; ++kb)
#pragma unroll
                for (int r = 0; r < 16; ++r) mx = fmaxf(mx, sacc[kb][r]);
            mx = max_halves(mx);
            const float m_new = fmaxf(m, mx * c);
            // A row with no admitted key yet keeps m = -inf; exponents use 0.
            const float m_use = (m_new == kNegInf) ? 0.0f : m_new;
            const float alpha = exp2_fast(m - m_use);
            m = m_new;
            const float neg_m = -m_use;
            // P = 2^(S c - m'), the row's partial sum, and P^T packed as the
            // B operand of the four 16-key k-steps.
            half8 pb[4];
            float psum = 0.0f;
#pragma unroll
            for (int kb = 0; kb < 2; ++kb)
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    float p = exp2_fast(__builtin_fmaf(sacc[kb][r], c, neg_m));
                    psum += p;
                    pb[2 * kb + (r >> 3)][r & 7] = to_half(p);
                }
            lsum = lsum * alpha + psum;
#pragma unroll
            for (int db = 0; db < 2; ++db)
#pragma unroll
                for (int r = 0; r < 16; ++r) oacc[db][r] *= alpha;
            // O^T += V^T P^T.  k-step s covers the tile's keys 16 s + 4 hi
            // + 0..3 and 16 s + 8 + 4 hi + 0..3 (the accumulator's order).
#pragma unroll
            for (int s = 0; s < 4; ++s) {
#pragma unroll
                for (int db = 0; db < 2; ++db) {
                    const half_t* vrow = Vs + (32 * db + l32) * kLdsRow + 16 * s + 4 * hi;
                    half8 a = cat(*(const half4*)vrow, *(const half4*)(vrow + 8));
                    oacc[db] = mfma32(a, pb[s], oacc[db]);
                }
            }
        }

        if (j + 1 < n_kt) store_tile(j + 1, buf ^ 1);
        __syncthreads();
    }

    if (!wave_rows) return;
    // Epilogue: l over both halves, O / l, L = m + log2 l; rows with no
    // admitted key (l = 0) get O = 0 and L = -inf.
    const float l_tot = sum_halves(lsum);
    const bool empty = !(l_tot > 0.0f);
    const float inv = empty ? 0.0f : rcp_fast(l_tot);
    half_t* op = O + (((size_t)b * T + q) * H + h) * kHeadDim;
#pragma unroll
    for (int db = 0; db < 2; ++db)
#pragma unroll
        for (int rg = 0; rg < 4; ++rg) {
            half4 v;
#pragma unroll
            for (int e = 0; e < 4; ++e) v[e] = to_half(oacc[db][4 * rg + e] * inv);
            *(half4*)(op + 32 * db + 8 * rg + 4 * hi) = v;
        }
    if (hi == 0) L[((size_t)b * H + h) * T + q] = empty ? kNegInf : m + log2_fast(l_tot);
}

}  // namespace

size_t forward_blocks(const Shape& sh) {
    return (size_t)((sh.T + kFwdRows - 1) / kFwdRows) * sh.batch * sh.heads;
}

hipError_t launch_forward(const Shape& sh, const void* Q, const void* K, const void* Vt, void* O, float* L,
                          float c, hipStream_t stream) {
    const int n_qtiles = (sh.T + kFwdRows - 1) / kFwdRows;
    const int BH = sh.batch * sh.heads;
    dim3 grid((unsigned)(n_qtiles * BH)), block(kFwdThreads);
    auto args = [&](auto kern) {
        hipLaunchKernelGGL(kern, grid, block, 0, stream, (const half_t*)Q, (const half_t*)K, (const half_t*)Vt,
                           (half_t*)O, L, sh.seqlens, c, sh.T, sh.heads, sh.kv_heads, n_qtiles, BH,
                           sh.block_order);
    };
    const bool varlen = sh.seqlens != nullptr;
    if (sh.causal) {
        if (varlen) args(sa_forward_kernel<true, true>);
        else args(sa_forward_kernel<true, false>);
    } else {
        if (varlen) args(sa_forward_kernel<false, true>);
        else args(sa_forward_kernel<false, false>);
    }
    return hipGetLastError();
}

}  // namespace sa
