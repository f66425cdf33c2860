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

// Zero the halves of an 8-half chunk at positions >= keep (keep may be <= 0 or >= 8).
__device__ __forceinline__ uint4 clear_tail(uint4 v, int keep) {
    uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
    for (int t = 0; t < 8; ++t)
        if (t >= keep) w[t >> 1] &= (t & 1) ? 0x0000ffffu : 0xffff0000u;
    return make_uint4(w[0], w[1], w[2], w[3]);
}

template <bool CAUSAL, bool VARLEN>
__global__ __launch_bounds__(kFwdThreads, 2) void sa_forward_kernel(
    const half_t* __restrict__ Q, const half_t* __restrict__ K, const half_t* __restrict__ Vt,
    half_t* __restrict__ O, float* __restrict__ L, const int32_t* __restrict__ seqlens, float c, int T,
    int H, int KV, int n_qtiles, int BH, int block_order) {
    __shared__ __attribute__((aligned(16))) half_t lds[2][2][kTileHalves];  // [buffer][K | V^T][row][col]

    const int tid = threadIdx.x, lane = tid & 63, wave = wave_id();
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
    const int qw = q0 + 32 * wave;                 // this wave's first query (scalar)
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

    f32x16 oacc0 = zero16(), oacc1 = zero16();  // O^T, d blocks 0..31 and 32..63
    float m = kNegInf, lsum = 0.0f;

    // Staging: 512 16-byte chunks per 64x64 tile; thread tid moves chunks
    // tid and tid + 256 of K and of V^T.
    const int row_a = tid >> 3, row_b = row_a + 32, col8 = (tid & 7) * 8;
    uint4 ka, kb, va, vb;
#define SA_FWD_LOAD(j)                                                                      \
    do {                                                                                    \
        const half_t* kt_ = Kp + (size_t)((j) * kTile) * kHeadDim;                          \
        ka = *(const uint4*)(kt_ + row_a * kHeadDim + col8);                                \
        kb = *(const uint4*)(kt_ + row_b * kHeadDim + col8);                                \
        va = *(const uint4*)(Vp + (size_t)row_a * T + (j) * kTile + col8);                  \
        vb = *(const uint4*)(Vp + (size_t)row_b * T + (j) * kTile + col8);                  \
    } while (0)
#define SA_FWD_STORE(j, buf)                                                                \
    do {                                                                                    \
        if (VARLEN && (j) * kTile + col8 + 8 > len) {                                       \
            /* keys at or past the length carry P = 0: clear their V entries */             \
            va = clear_tail(va, len - ((j) * kTile + col8));                                \
            vb = clear_tail(vb, len - ((j) * kTile + col8));                                \
        }                                                                                   \
        *(uint4*)&lds[buf][0][row_a * kLdsRow + col8] = ka;                                 \
        *(uint4*)&lds[buf][0][row_b * kLdsRow + col8] = kb;                                 \
        *(uint4*)&lds[buf][1][row_a * kLdsRow + col8] = va;                                 \
        *(uint4*)&lds[buf][1][row_b * kLdsRow + col8] = vb;                                 \
    } while (0)

    if (n_kt > 0) {
        SA_FWD_LOAD(0);
        SA_FWD_STORE(0, 0);
    }
    __syncthreads();

    for (int j = 0; j < n_kt; ++j) {
        const int buf = j & 1;
        if (j + 1 < n_kt) SA_FWD_LOAD(j + 1);

        if (wave_live && j * kTile < kend_w) {
            const half_t* Ks = lds[buf][0];
            const half_t* Vs = lds[buf][1];
            // S^T = K Q^T for the tile's two 32-key blocks.
            f32x16 s0 = zero16(), s1 = zero16();
#pragma unroll
            for (int s = 0; s < 4; ++s) {
                half8 a0 = *(const half8*)(Ks + l32 * kLdsRow + 16 * s + 8 * hi);
                half8 a1 = *(const half8*)(Ks + (32 + l32) * kLdsRow + 16 * s + 8 * hi);
                s0 = mfma32(a0, qf[s], s0);
                s1 = mfma32(a1, qf[s], s1);
            }
            // Mask: key past the query (causal) or at/past the length; only
            // tiles that reach past the wave's first query or the length.
            const int key0 = j * kTile;
            const bool need_mask = (CAUSAL && key0 + kTile - 1 > qw) ||
                                   (VARLEN && (key0 + kTile > len || qw + 32 > len));
            if (need_mask) {
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    const int k0 = key0 + 8 * (r >> 2) + 4 * hi + (r & 3), k1 = k0 + 32;
                    const bool m0 = (CAUSAL && k0 > q) || (VARLEN && (k0 >= len || q >= len));
                    const bool m1 = (CAUSAL && k1 > q) || (VARLEN && (k1 >= len || q >= len));
                    s0[r] = m0 ? kNegInf : s0[r];
                    s1[r] = m1 ? kNegInf : s1[r];
                }
            }
            // Row maximum of the raw scores (c > 0, so max(S) c = max(S c)).
            float mx = fmaxf(s0[0], s1[0]);
#pragma unroll
            for (int r = 1; r < 16; ++r) mx = fmaxf(mx, fmaxf(s0[r], s1[r]));
            mx = max_halves(mx);
            const float m_new = fmaxf(m, mx * c);
            // A row with no admitted key yet keeps m = -inf; exponents use 0.
            const float m_use = (m_new == kNegInf) ? 0.0f : m_new;
            const float neg_m = -m_use;
            // P = 2^(S c - m'), the row's partial sum, and P^T packed as the
            // B operand of the four 16-key k-steps (k-step s: block s / 2,
            // accumulator rows 8 (s % 2) .. + 7).
            uint32_t w[16];
            float psum = 0.0f;
#pragma unroll
            for (int r = 0; r < 16; r += 2) {
                const float p0 = exp2_fast(__builtin_fmaf(s0[r], c, neg_m));
                const float p1 = exp2_fast(__builtin_fmaf(s0[r + 1], c, neg_m));
                const float p2 = exp2_fast(__builtin_fmaf(s1[r], c, neg_m));
                const float p3 = exp2_fast(__builtin_fmaf(s1[r + 1], c, neg_m));
                psum += (p0 + p1) + (p2 + p3);
                w[r >> 1] = pack_half2(p0, p1);
                w[8 + (r >> 1)] = pack_half2(p2, p3);
            }
            // Rescale l and O when some row's maximum grew (2^(m - m') = 1 otherwise).
            if (__builtin_amdgcn_ballot_w64(m_new != m) != 0) {
                const float alpha = exp2_fast(m - m_use);
                lsum *= alpha;
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    oacc0[r] *= alpha;
                    oacc1[r] *= alpha;
                }
            }
            lsum += psum;
            m = m_new;
            // O^T += V^T P^T.  k-step s covers the tile's keys 16 s + 4 hi
            // + 0..3 and 16 s + 8 + 4 hi + 0..3 (the accumulator's order).
#pragma unroll
            for (int s = 0; s < 4; ++s) {
                const half8 pb = half8_from_words(w[4 * s], w[4 * s + 1], w[4 * s + 2], w[4 * s + 3]);
                const half_t* v0 = Vs + l32 * kLdsRow + 16 * s + 4 * hi;
                const half_t* v1 = v0 + 32 * kLdsRow;
                oacc0 = mfma32(cat(*(const half4*)v0, *(const half4*)(v0 + 8)), pb, oacc0);
                oacc1 = mfma32(cat(*(const half4*)v1, *(const half4*)(v1 + 8)), pb, oacc1);
            }
        }

        if (j + 1 < n_kt) SA_FWD_STORE(j + 1, buf ^ 1);
        __syncthreads();
    }
#undef SA_FWD_LOAD
#undef SA_FWD_STORE

    if (!wave_rows) return;
    // Epilogue: l over both halves, O / l, L = m + log2 l; rows with no
    // admitted key (l = 0) get O = 0 and L = -inf.  O goes through this
    // wave's own LDS rows so that the stores are whole 128-byte rows.
    const float l_tot = sum_halves(lsum);
    const bool empty = !(l_tot > 0.0f);
    const float inv = empty ? 0.0f : rcp_fast(l_tot);
    half_t* ow = &lds[0][0][0] + wave * 32 * kLdsRow;  // 32 rows x 72 halves per wave
#pragma unroll
    for (int rg = 0; rg < 4; ++rg) {
        uint2 v0 = make_uint2(pack_half2(oacc0[4 * rg] * inv, oacc0[4 * rg + 1] * inv),
                              pack_half2(oacc0[4 * rg + 2] * inv, oacc0[4 * rg + 3] * inv));
        uint2 v1 = make_uint2(pack_half2(oacc1[4 * rg] * inv, oacc1[4 * rg + 1] * inv),
                              pack_half2(oacc1[4 * rg + 2] * inv, oacc1[4 * rg + 3] * inv));
        *(uint2*)(ow + l32 * kLdsRow + 8 * rg + 4 * hi) = v0;
        *(uint2*)(ow + l32 * kLdsRow + 32 + 8 * rg + 4 * hi) = v1;
    }
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    // 32 rows x 8 chunks of 16 bytes: 4 chunks per lane.
#pragma unroll
    for (int u = 0; u < 4; ++u) {
        const int chunk = lane + 64 * u, row = chunk >> 3, col = (chunk & 7) * 8;
        const uint4 v = *(const uint4*)(ow + row * kLdsRow + col);
        *(uint4*)(O + (((size_t)b * T + qw + row) * H + h) * kHeadDim + col) = v;
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
