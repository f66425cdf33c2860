// sa_query.hip -- the query pass of the two-launch backward on gfx950.
//
// Method: StreamingAttentionSM86 page, banner "The backward pass,
// deterministic and in two launches (no atomics)", the query launch: a block
// per query tile of a query head forms D = rowsum(dO * O) for its rows (and
// writes it for the key launch), then walks the key tiles up to the diagonal
// as the forward does, recomputing per tile
//   S = Q K^T,  P = 2^(S c - L),  dP = dO V^T,  dS = P (dP - D),
// and keeping dQ = s * sum over the tiles of dS K.  No score gradient leaves
// the chip: the key launch (the key pass without its dS store) forms dK and
// dV the same way.
//
// MI355X design: a 256-thread workgroup (4 wave64s) takes 128 queries of one
// query head, each wave 32 queries, and walks the key tiles with the K tile
// and the V^T tile (or, with V as rows, the V row tile, staged and read like
// K's) staged once in LDS for the four waves (16-byte loads one tile ahead,
// double-buffered).  Per tile a wave runs 24 products on
// v_mfma_f32_32x32x16_f16, all in the forward's orientation (lane = query):
//   S^T  = K Q^T    (A = K rows, LDS; B = Q^T, registers)
//   dP^T = V dO^T   (A = V rows, read transposed from the V^T tile; B = dO^T)
//   dQ^T += K^T dS^T (A = K^T, read transposed from the K tile in the permuted
//                     key order of the score accumulator; B = dS^T packed to
//                     binary16 straight from the accumulator, as the forward
//                     feeds P to P V)
// so P, dP and dS never leave registers.  A tile's dQ products are issued
// one tile late, spread through the next tile's vector work at raised wave
// priority (K tiles in a three-slot ring so the late reads stay valid).  Both tiles are stored unpadded
// with the 16-byte chunks of each row permuted (swz), which keeps the row
// reads and the transposed reads free of bank conflicts.
#include <type_traits>

#include "sa_device.h"
#include "sa_internal.h"

namespace sa {

namespace {

constexpr int kQpWaves = 4;
constexpr int kQpRows = 32 * kQpWaves;       // queries per workgroup
constexpr int kQpThreads = 64 * kQpWaves;
constexpr int kQpTile = kTile * kHeadDim;    // one unpadded 64x64 tile

// Row r's 16-byte chunk c of a staged tile sits at chunk c ^ key(r).  LDS
// moves 256 bytes (64 banks) a cycle, two 128-byte rows side by side: a
// 16-byte row read by 16 lanes (16 consecutive rows, one chunk) meets no bank
// conflict when key is distinct over the 8 rows of each parity among them
// (key takes bits 1..3 of r), and a transposed read of 4 rows x 2 chunks of
// an aligned group of 4 rows none when the two rows of a parity land in
// different 4-chunk halves (bit 2 of key is bit 1 of r).
__device__ __forceinline__ int qp_key(int row) { return (((row >> 1) & 1) << 2) | ((row >> 2) & 3); }
__device__ __forceinline__ int qp_swz(int row, int col) {
    return row * kHeadDim + (((col >> 3) ^ qp_key(row)) << 3) + (col & 7);
}
// The element a transposed read names so that lane l receives column
// col0 + l % 32 at rows row0 + 0..3 (row0 = rowA for lanes 0..31, rowB for
// 32..63) of a staged tile.
__device__ __forceinline__ int qp_tr(int lane, int rowA, int rowB, int col0) {
    const int row = ((lane & 32) ? rowB : rowA) + ((lane & 15) >> 2);
    return qp_swz(row, col0 + 16 * ((lane >> 4) & 1) + 4 * (lane & 3));
}

// Zero the halves of an 8-half chunk at positions >= keep (keep may be <= 0 or >= 8).
__device__ __forceinline__ uint4 qp_clear_tail(uint4 v, int keep) {
    uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
    for (int t = 0; t < 8; ++t)
        if (t >= keep) w[t >> 1] &= (t & 1) ? 0x0000ffffu : 0xffff0000u;
    return make_uint4(w[0], w[1], w[2], w[3]);
}

// Issue-order hint for one tile: the previous tile's 8 dQ products spread
// through this tile's exponentials and dS arithmetic.
#define SA_QP_SGB(mask, n) __builtin_amdgcn_sched_group_barrier(mask, n, 0)
#define SA_QP_SLOT SA_QP_SGB(0x008, 1); SA_QP_SGB(0x002, 12)
#define SA_QP_INTERLEAVE()                                    \
    do {                                                      \
        SA_QP_SLOT; SA_QP_SLOT; SA_QP_SLOT; SA_QP_SLOT;       \
        SA_QP_SLOT; SA_QP_SLOT; SA_QP_SLOT; SA_QP_SLOT;       \
    } while (0)

template <bool CAUSAL, bool VARLEN, bool VROWS>
__global__ __launch_bounds__(kQpThreads, 2) void sa_query_kernel(
    const half_t* __restrict__ Q, const half_t* __restrict__ K, const half_t* __restrict__ Vt,
    const half_t* __restrict__ dO, const half_t* __restrict__ O, const float* __restrict__ L,
    float* __restrict__ D, float* __restrict__ dQ, const int32_t* __restrict__ seqlens, float c, float s,
    int T, int H, int KV, int n_qtiles, int BH, int block_order, ProjectionOut qproj) {
    // K tile j lives in buffer j % 3: its dQ products are issued one tile late,
    // beside the next tile's vector work, while tile j + 1 is staged.
    __shared__ __attribute__((aligned(16))) half_t kls[3][kQpTile];  // K tiles [key][d]
    __shared__ __attribute__((aligned(16))) half_t vls[2][kQpTile];  // V^T tiles [d][key] (VROWS: V [key][d])

    const int tid = threadIdx.x, lane = tid & 63, wave = wave_id();
    const int l32 = lane & 31, hi = lane >> 5;

    // Block -> (batch*head, query tiles): as the forward, the pair (n - 1 - p,
    // p) of equal causal length with the heads of one kv head on one XCD
    // (order 0), or one tile per block in plain order (order 1).
    int bh, n_items, items[2];
    if (VARLEN && block_order != kOrderPlain && BH / H <= kMaxRankedBatch) {
        // Variable lengths: the longest sequences' blocks first, then the
        // schedule's order within each sequence.
        const int per_b = H * (block_order == kOrderPairs ? (n_qtiles + 1) / 2 : n_qtiles);
        const int r = (int)blockIdx.x / per_b, rest = (int)blockIdx.x % per_b, k = rest / H;
        bh = batch_of_rank(seqlens, BH / H, T, r) * H + rest % H;
        items[0] = n_qtiles - 1 - k;
        items[1] = k;
        n_items = (block_order == kOrderPairs && k < items[0]) ? 2 : 1;
    } else if (block_order == kOrderPairs) {
        int pair;
        pair_schedule((int)blockIdx.x, (BH / H) * KV, H / KV, pair, bh);
        items[0] = n_qtiles - 1 - pair;
        items[1] = pair;
        n_items = pair < items[0] ? 2 : 1;
    } else if (block_order == kOrderSingle) {  // one tile per block, the longest first
        items[0] = items[1] = n_qtiles - 1 - (int)(blockIdx.x / BH);
        bh = (int)(blockIdx.x % BH);
        n_items = 1;
    } else {
        items[0] = items[1] = (int)(blockIdx.x % n_qtiles);
        bh = (int)(blockIdx.x / n_qtiles);
        n_items = 1;
    }
    const int b = bh / H, h = bh % H, kv = h / (H / KV);
    const int len = VARLEN ? min(max(seqlens[b], 0), T) : T;
    const size_t kv_off = ((size_t)b * KV + kv) * (size_t)T * kHeadDim;
    const half_t* Kp = K + kv_off;
    const half_t* Vp = Vt + kv_off;

    // Staging: thread tid moves 16-byte chunks (row_a, cc) and (row_a + 32, cc)
    // of a K tile (rows = keys) and of a V^T tile (rows = d, columns = keys),
    // or of a V row tile, staged exactly like K's.  Buffer loads over the
    // (batch, kv head) slice: a fixed per-lane register offset and a scalar
    // tile offset, so the loop forms no addresses on the vector unit.
    const int row_a = tid >> 3, row_b = row_a + 32, cc = tid & 7;
    const int slice_bytes = T * kHeadDim * 2;
    const __amdgpu_buffer_rsrc_t k_rsrc =
        __builtin_amdgcn_make_buffer_rsrc((void*)Kp, (short)0, slice_bytes, kBufferRsrcWord3);
    const __amdgpu_buffer_rsrc_t v_rsrc =
        __builtin_amdgcn_make_buffer_rsrc((void*)Vp, (short)0, slice_bytes, kBufferRsrcWord3);
    const int k_off_a = (row_a * kHeadDim + cc * 8) * 2, k_off_b = (row_b * kHeadDim + cc * 8) * 2;
    const int v_off_a = VROWS ? k_off_a : (row_a * T + cc * 8) * 2;
    const int v_off_b = VROWS ? k_off_b : (row_b * T + cc * 8) * 2;
    auto load = [&](int j, uint4& ka, uint4& kb, uint4& va, uint4& vb) {
        const int ktile = j * kTile * kHeadDim * 2, vtile = VROWS ? ktile : j * kTile * 2;
        ka = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(k_rsrc, k_off_a, ktile, 0));
        kb = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(k_rsrc, k_off_b, ktile, 0));
        va = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(v_rsrc, v_off_a, vtile, 0));
        vb = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(v_rsrc, v_off_b, vtile, 0));
    };
    auto store = [&](int j, int kbuf, int buf, uint4 ka, uint4 kb, uint4 va, uint4 vb) {
        if (VARLEN) {
            // keys at or past the length: P and dS are masked to zero, and
            // their K rows and V^T columns are cleared so that no padding
            // value reaches a product
            if (j * kTile + row_a >= len) ka = make_uint4(0, 0, 0, 0);
            if (j * kTile + row_b >= len) kb = make_uint4(0, 0, 0, 0);
            if (VROWS) {
                if (j * kTile + row_a >= len) va = make_uint4(0, 0, 0, 0);
                if (j * kTile + row_b >= len) vb = make_uint4(0, 0, 0, 0);
            } else if (j * kTile + cc * 8 + 8 > len) {
                va = qp_clear_tail(va, len - (j * kTile + cc * 8));
                vb = qp_clear_tail(vb, len - (j * kTile + cc * 8));
            }
        }
        *(uint4*)&kls[kbuf][qp_swz(row_a, cc * 8)] = ka;
        *(uint4*)&kls[kbuf][qp_swz(row_b, cc * 8)] = kb;
        *(uint4*)&vls[buf][qp_swz(row_a, cc * 8)] = va;
        *(uint4*)&vls[buf][qp_swz(row_b, cc * 8)] = vb;
    };

    auto process = [&](const int qtile) {
        const int q0 = qtile * kQpRows;
        const int qw = q0 + 32 * wave;          // this wave's first query
        const int q = qw + l32;                 // this lane's query
        const bool wave_rows = qw < T;          // T % 64 == 0: whole wave in or out
        const int row_limit = VARLEN ? len : T;
        int kend = CAUSAL ? min(q0 + kQpRows, T) : T;
        if (VARLEN) kend = min(kend, len);
        if (VARLEN && q0 >= len) kend = 0;  // every row is padding: no key tile to walk
        const int n_kt = (kend + kTile - 1) / kTile;
        int kend_w = CAUSAL ? qw + 32 : T;
        if (VARLEN) kend_w = min(kend_w, len);
        const bool wave_live = wave_rows && qw < row_limit;
        const int n_kt_w = wave_live ? min((kend_w + kTile - 1) / kTile, n_kt) : 0;

        // Q^T and dO^T as B operands: lane (query l32, half hi) holds
        // Q[q][16 t + 8 hi + 0..7] and dO[q][16 t + 8 hi + 0..7], t = 0..3.
        const size_t row_id = ((size_t)b * H + h) * T + q;
        half8 qf[4], of[4];
        float Dq = 0.0f, negL = 0.0f;
        if (wave_live) {
            const half_t* qp = Q + row_id * kHeadDim + 8 * hi;
            const half_t* op = dO + row_id * kHeadDim + 8 * hi;
#pragma unroll
            for (int t = 0; t < 4; ++t) {
                qf[t] = *(const half8*)(qp + 16 * t);
                of[t] = *(const half8*)(op + 16 * t);
            }
        }
        if (wave_rows) {
            // D = rowsum(dO * O) over this lane's 32 columns, then both halves;
            // binary32, every fp16 widened, fused multiply-adds.  O is the
            // forward's (token-major) output.
            float part = 0.0f;
            if (wave_live) {
                const half_t* orow = O + (((size_t)b * T + q) * H + h) * kHeadDim + 8 * hi;
#pragma unroll
                for (int t = 0; t < 4; ++t) {
                    const half8 o8 = *(const half8*)(orow + 16 * t);
#pragma unroll
                    for (int e = 0; e < 8; ++e) part = __builtin_fmaf((float)of[t][e], (float)o8[e], part);
                }
            }
            Dq = sum_halves(part);
            if (VARLEN && q >= len) Dq = 0.0f;
            if (hi == 0) D[row_id] = Dq;
            negL = (VARLEN && q >= len) ? 0.0f : -L[row_id];
        }

        f32x16 dq0 = zero16(), dq1 = zero16();  // dQ^T, d blocks 0..31 and 32..63
        if (n_kt > 0) {
            uint4 ka, kb, va, vb;
            load(0, ka, kb, va, vb);
            store(0, 0, 0, ka, kb, va, vb);
        }
        __syncthreads();
        vm_wait_all();  // the staged tile and Q, dO have landed (see the forward)

        // dQ^T += K^T dS^T for one tile.  k-step t covers the tile's keys
        // 16 t + 4 hi + 0..3 and 16 t + 8 + 4 hi + 0..3 (the accumulator's
        // order); K^T's A operand is read transposed in that same order.
        auto dq_products = [&](const half_t* Ks, const uint32_t (&w)[16]) {
#pragma unroll
            for (int t = 0; t < 4; ++t) {
                const half8 pb = half8_from_words(w[4 * t], w[4 * t + 1], w[4 * t + 2], w[4 * t + 3]);
                const half8 k0 = cat(lds_read_tr(Ks + qp_tr(lane, 16 * t, 16 * t + 4, 0)),
                                     lds_read_tr(Ks + qp_tr(lane, 16 * t + 8, 16 * t + 12, 0)));
                const half8 k1 = cat(lds_read_tr(Ks + qp_tr(lane, 16 * t, 16 * t + 4, 32)),
                                     lds_read_tr(Ks + qp_tr(lane, 16 * t + 8, 16 * t + 12, 32)));
                dq0 = mfma32(k0, pb, dq0);
                dq1 = mfma32(k1, pb, dq1);
            }
        };

        // dS of the previous tile, packed (the B operand of its dQ products).
        // Before the first tile it is zero and tile 0's K (finite) stands in,
        // so those products add exact zeros.
        uint32_t wprev[16];
#pragma unroll
        for (int i = 0; i < 16; ++i) wprev[i] = 0u;
        int kcur = 0, kprev = 0;  // ring positions of K tiles j and j - 1
        for (int j = 0; j < n_kt; ++j) {
            const int buf = j & 1;
            const bool more = j + 1 < n_kt;
            const int knext = kcur == 2 ? 0 : kcur + 1;
            uint4 ka, kb, va, vb;
            if (more) load(j + 1, ka, kb, va, vb);
            if (j < n_kt_w) {
                __builtin_amdgcn_s_setprio(1);
                const half_t* Ks = kls[kcur];
                const half_t* Vs = vls[buf];
                // S^T = K Q^T and dP^T = V dO^T for the tile's two 32-key blocks.
                f32x16 s0 = zero16(), s1 = zero16(), p0 = zero16(), p1 = zero16();
#pragma unroll
                for (int t = 0; t < 4; ++t) {
                    const half8 a0 = *(const half8*)(Ks + qp_swz(l32, 16 * t + 8 * hi));
                    const half8 a1 = *(const half8*)(Ks + qp_swz(32 + l32, 16 * t + 8 * hi));
                    s0 = mfma32(a0, qf[t], s0);
                    s1 = mfma32(a1, qf[t], s1);
                    // A = V: lane (key, hi) holds V^T[16 t + 8 hi + 0..7][key],
                    // a row read of a V row tile or a transposed read of V^T's.
                    half8 v0, v1;
                    if (VROWS) {
                        v0 = *(const half8*)(Vs + qp_swz(l32, 16 * t + 8 * hi));
                        v1 = *(const half8*)(Vs + qp_swz(32 + l32, 16 * t + 8 * hi));
                    } else {
                        v0 = cat(lds_read_tr(Vs + qp_tr(lane, 16 * t, 16 * t + 8, 0)),
                                 lds_read_tr(Vs + qp_tr(lane, 16 * t + 4, 16 * t + 12, 0)));
                        v1 = cat(lds_read_tr(Vs + qp_tr(lane, 16 * t, 16 * t + 8, 32)),
                                 lds_read_tr(Vs + qp_tr(lane, 16 * t + 4, 16 * t + 12, 32)));
                    }
                    p0 = mfma32(v0, of[t], p0);
                    p1 = mfma32(v1, of[t], p1);
                }
                // The previous tile's dQ products go into the matrix pipe
                // behind these, spread through this tile's vector work.
                __builtin_amdgcn_sched_barrier(0);
                dq_products(kls[j == 0 ? kcur : kprev], wprev);
                // P = 2^(S c - L), dS = P (dP - D); masked elements are
                // selected to exact zeros (never multiplied: padding may hold
                // anything).  Lane holds key 8 (r / 4) + 4 hi + r % 4 (+ 32 for
                // the second block) of query q.
                float g0[16], g1[16];
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    g0[r] = exp2_fast(__builtin_fmaf(s0[r], c, negL)) * (p0[r] - Dq);
                    g1[r] = exp2_fast(__builtin_fmaf(s1[r], c, negL)) * (p1[r] - Dq);
                }
                SA_QP_INTERLEAVE();
                __builtin_amdgcn_s_setprio(0);
                const int key0 = j * kTile;
                const bool need_mask = (CAUSAL && key0 + kTile - 1 > qw) ||
                                       (VARLEN && (key0 + kTile > len || qw + 32 > len));
                if (need_mask) {
#pragma unroll
                    for (int r = 0; r < 16; ++r) {
                        const int k0 = key0 + 8 * (r >> 2) + 4 * hi + (r & 3), k1 = k0 + 32;
                        const bool m0 = (CAUSAL && k0 > q) || (VARLEN && (k0 >= len || q >= len));
                        const bool m1 = (CAUSAL && k1 > q) || (VARLEN && (k1 >= len || q >= len));
                        g0[r] = m0 ? 0.0f : g0[r];
                        g1[r] = m1 ? 0.0f : g1[r];
                    }
                }
#pragma unroll
                for (int i = 0; i < 8; ++i) {
                    wprev[i] = pack_half2(g0[2 * i], g0[2 * i + 1]);
                    wprev[8 + i] = pack_half2(g1[2 * i], g1[2 * i + 1]);
                }
            } else if (j == n_kt_w && j > 0) {
                // The wave's last tile's products (its K tile is not restaged
                // before the next step ends).
                dq_products(kls[kprev], wprev);
            }
            // Tile j + 1 goes to K ring slot j + 1 (which held tile j - 2,
            // last read in the previous step) and V buffer buf ^ 1.
            if (more) store(j + 1, knext, buf ^ 1, ka, kb, va, vb);
            vm_wait_all();  // nothing is outstanding here; keeps the compiler's count exact
            __syncthreads();
            kprev = kcur;
            kcur = knext;
        }
        // A wave that formed the last tile adds its products here.
        if (n_kt_w == n_kt && n_kt > 0) dq_products(kls[kprev], wprev);

        if (!wave_rows) return;
        // dQ = s dQ^T: lane holds d = 8 (r / 4) + 4 hi + r % 4 of query q.
        const float scale = (!VARLEN || q < len) ? s : 0.0f;
        if (qproj.f32) {
            // Projection variant (same page, the shared query pass stored
            // straight into a fused projection's gradient): row q of the
            // token-major gradient, columns 64 h + d, binary32 and bfloat16.
            const size_t at = ((size_t)b * T + q) * (size_t)qproj.width + kHeadDim * h;
#pragma unroll
            for (int rg = 0; rg < 4; ++rg) {
                const int c0 = 8 * rg + 4 * hi;
                f32x4 v0 = {dq0[4 * rg], dq0[4 * rg + 1], dq0[4 * rg + 2], dq0[4 * rg + 3]};
                f32x4 v1 = {dq1[4 * rg], dq1[4 * rg + 1], dq1[4 * rg + 2], dq1[4 * rg + 3]};
                v0 *= scale;
                v1 *= scale;
                *(f32x4*)(qproj.f32 + at + c0) = v0;
                *(f32x4*)(qproj.f32 + at + 32 + c0) = v1;
                *(uint2*)(qproj.b16 + at + c0) = pack_bf16x4(v0[0], v0[1], v0[2], v0[3]);
                *(uint2*)(qproj.b16 + at + 32 + c0) = pack_bf16x4(v1[0], v1[1], v1[2], v1[3]);
            }
            return;
        }
        float* dq = dQ + row_id * kHeadDim;
#pragma unroll
        for (int rg = 0; rg < 4; ++rg) {
            f32x4 v0 = {dq0[4 * rg], dq0[4 * rg + 1], dq0[4 * rg + 2], dq0[4 * rg + 3]};
            f32x4 v1 = {dq1[4 * rg], dq1[4 * rg + 1], dq1[4 * rg + 2], dq1[4 * rg + 3]};
            *(f32x4*)(dq + 8 * rg + 4 * hi) = v0 * scale;
            *(f32x4*)(dq + 32 + 8 * rg + 4 * hi) = v1 * scale;
        }
    };
    process(items[0]);
    if (n_items == 2) {
        __syncthreads();  // every wave is past the first item's last tile reads
        process(items[1]);
    }
}

}  // namespace

int query_order(const Shape& sh) {
    return tile_schedule(sh, (size_t)sh.batch * sh.heads, (sh.T + kQpRows - 1) / kQpRows);
}
size_t query_pass_blocks(const Shape& sh) {
    return tile_schedule_blocks(query_order(sh), (size_t)sh.batch * sh.heads, (sh.T + kQpRows - 1) / kQpRows);
}

hipError_t launch_query_pass_to(const Shape& sh, const void* dO, const void* O, const float* L, const void* Q,
                                const void* K, const void* Vt, float c, float s, float* D, float* dQ,
                                const ProjectionOut& qproj, hipStream_t stream) {
    const int n_qtiles = (sh.T + kQpRows - 1) / kQpRows;
    const int BH = sh.batch * sh.heads;
    dim3 grid((unsigned)query_pass_blocks(sh)), block(kQpThreads);
    auto go = [&](auto kern) {
        hipLaunchKernelGGL(kern, grid, block, 0, stream, (const half_t*)Q, (const half_t*)K, (const half_t*)Vt,
                           (const half_t*)dO, (const half_t*)O, L, D, dQ, sh.seqlens, c, s, sh.T, sh.heads,
                           sh.kv_heads, n_qtiles, BH, query_order(sh), qproj);
    };
    const bool varlen = sh.seqlens != nullptr;
    auto pick = [&](auto rows_tag) {
        constexpr bool R = decltype(rows_tag)::value;
        if (sh.causal) {
            if (varlen) go(sa_query_kernel<true, true, R>);
            else go(sa_query_kernel<true, false, R>);
        } else {
            if (varlen) go(sa_query_kernel<false, true, R>);
            else go(sa_query_kernel<false, false, R>);
        }
    };
    if (sh.v_rows) pick(std::true_type{});
    else pick(std::false_type{});
    return hipGetLastError();
}

hipError_t launch_query_pass(const Shape& sh, const void* dO, const void* O, const float* L, const void* Q,
                             const void* K, const void* Vt, float c, float s, float* D, float* dQ,
                             hipStream_t stream) {
    return launch_query_pass_to(sh, dO, O, L, Q, K, Vt, c, s, D, dQ, ProjectionOut{nullptr, nullptr, 0}, stream);
}

hipError_t launch_query_pass_projection(const Shape& sh, const void* dO, const void* O, const float* L,
                                        const void* Q, const void* K, const void* Vt, float c, float s, float* D,
                                        const ProjectionOut& qproj, hipStream_t stream) {
    return launch_query_pass_to(sh, dO, O, L, Q, K, Vt, c, s, D, nullptr, qproj, stream);
}

}  // namespace sa
