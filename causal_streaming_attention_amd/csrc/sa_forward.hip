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
// tile's K rows and V^T rows (or V rows, when V comes as rows [T][64]: its
// tile is then read transposed) are staged once in LDS for all four waves
// with coalesced 16-byte loads (K two tiles ahead, V one tile ahead).  A wave
// computes S^T = K Q^T with v_mfma_f32_32x32x16_f16 (A = K rows from LDS,
// B = the wave's Q kept in registers), so every lane holds 32 scores of ONE
// query: the row maximum is an in-lane max plus one v_permlane32_swap, the
// row sum stays a per-lane partial until the end (as the pages keep it per
// thread), and the rescale factor is per lane.  The fp16 P^T accumulators
// feed O^T += V^T P^T directly as the B operand: the contraction order over
// the tile's keys is permuted to match the accumulator layout, and V^T's A
// operand is read from LDS in the same permuted order, so P never leaves
// registers.
//
// The loop is software-pipelined: while tile j's softmax runs on the vector
// unit, the wave's matrix-core work is tile j + 1's scores and tile j - 1's
// P V, issued between the softmax instructions, at raised wave priority so
// that of the two waves on a SIMD the one with matrix work issues first.  P
// is first formed with the exponents' current maximum; the maximum is taken
// and moved (and P formed again) only on the wave's first tile and when some
// lane's sum of P exceeds 2^8, so P <= 2^8, the row maximum costs nothing on
// the other tiles and the O/l rescale is rare; O / l and L = m + log2 l are
// the same quantities whichever maximum the exponents used.  Blocks take
// the query tiles (n - 1 - p, p) in pairs of equal causal length, with the
// heads that share a kv head kept on one XCD (pair_schedule).
#include "sa_device.h"
#include <type_traits>

#include "sa_internal.h"

namespace sa {

namespace {

constexpr int kFwdWaves = 4;
constexpr int kFwdRows = 32 * kFwdWaves;     // queries per workgroup
constexpr int kFwdThreads = 64 * kFwdWaves;
constexpr int kTileHalves = kTile * kLdsRow; // one padded 64-row K tile in LDS
// V^T rows are padded to 68 halves (34 dwords): sixteen lanes reading 8 bytes
// from sixteen consecutive rows then touch 32 distinct banks.
constexpr int kVRow = 68;
constexpr int kVTileHalves = kTile * kVRow;
// A V row tile (V as rows [T][64]) is unpadded, 128-byte rows whose 16-byte
// chunk c sits at chunk c ^ vr_key(r): the transposed reads of P V's operand
// cover 4 rows x 2 chunks of an aligned group of 4 rows, and with bit 2 of
// the key equal to bit 1 of the row the two rows of each parity (which share
// banks, two 128-byte rows to the 256-byte bank row) land in different
// 4-chunk halves.
constexpr int kVRowsTileHalves = kTile * kHeadDim;
__device__ __forceinline__ int vr_key(int r) { return (((r >> 1) & 1) << 2) | ((r >> 2) & 3); }
__device__ __forceinline__ int vr_off(int r, int col) {
    return r * kHeadDim + (((col >> 3) ^ vr_key(r)) << 3) + (col & 7);
}
// The running maximum used for the exponents moves only when some lane's sum
// of its 32 P in a tile exceeds this bound (P >= 0, so then every P <= 2^8).
constexpr float kMaxSum = 256.0f;

// Zero the halves of an 8-half chunk at positions >= keep (keep may be <= 0 or >= 8).
__device__ __forceinline__ uint4 clear_tail(uint4 v, int keep) {
    uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
    for (int t = 0; t < 8; ++t)
        if (t >= keep) w[t >> 1] &= (t & 1) ? 0x0000ffffu : 0xffff0000u;
    return make_uint4(w[0], w[1], w[2], w[3]);
}

// Issue-order hints for one tile of the loop: the 16 products (8 for the next
// tile's scores, 8 for the previous tile's P V) spread through the softmax's
// vector work, with the LDS operand reads ahead of them.
#define SA_SGB(mask, n) __builtin_amdgcn_sched_group_barrier(mask, n, 0)
#define SA_FWD_SLOT_R SA_SGB(0x008, 1); SA_SGB(0x002, 6); SA_SGB(0x100, 1)
#define SA_FWD_SLOT SA_SGB(0x008, 1); SA_SGB(0x002, 6)
#define SA_FWD_INTERLEAVE()                                       \
    do {                                                          \
        SA_SGB(0x100, 8);                                         \
        SA_FWD_SLOT_R; SA_FWD_SLOT_R; SA_FWD_SLOT_R; SA_FWD_SLOT_R; \
        SA_FWD_SLOT_R; SA_FWD_SLOT_R; SA_FWD_SLOT_R; SA_FWD_SLOT_R; \
        SA_FWD_SLOT; SA_FWD_SLOT; SA_FWD_SLOT; SA_FWD_SLOT;       \
        SA_FWD_SLOT; SA_FWD_SLOT; SA_FWD_SLOT; SA_FWD_SLOT;       \
    } while (0)

template <bool CAUSAL, bool VARLEN, bool VROWS>
__global__ __launch_bounds__(kFwdThreads, 2) void sa_forward_kernel(
    const half_t* __restrict__ Q, const half_t* __restrict__ K, const half_t* __restrict__ Vt,
    half_t* __restrict__ O, float* __restrict__ L, const int32_t* __restrict__ seqlens, float c, int T,
    int H, int KV, int n_qtiles, int BH, int block_order) {
    // K tile j + 2 is staged while tile j + 1's scores are formed, and V^T
    // tile j + 1 while tile j - 1's products are summed: two K buffers and
    // three V^T buffers (V^T tile j lives in buffer j % 3).  VROWS: V comes
    // as rows [T][64] like K and its tiles are staged like K's.
    __shared__ __attribute__((aligned(16))) half_t kls[2][kTileHalves];
    __shared__ __attribute__((aligned(16))) half_t vls[3][VROWS ? kVRowsTileHalves : kVTileHalves];

    const int tid = threadIdx.x, lane = tid & 63, wave = wave_id();
    const int l32 = lane & 31, hi = lane >> 5;

    // Block -> (batch*head, query tiles).  Order 0: the pair of query tiles
    // (n - 1 - p, p), whose causal walks add up to the same length for every
    // p, with the heads of one kv head kept on one XCD.  Order 1: one query
    // tile per block in plain order.
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
    auto process = [&](const int qtile) {
    const int q0 = qtile * kFwdRows;
    const int qw = q0 + 32 * wave;                 // this wave's first query (scalar)
    const int q = qw + l32;                        // this lane's query
    const bool wave_rows = qw < T;                 // T % 64 == 0: whole wave in or out
    const int row_limit = VARLEN ? len : T;        // rows at or past it are masked

    // Key tiles the block walks, and the keys each wave needs.
    int kend = CAUSAL ? min(q0 + kFwdRows, T) : T;
    if (VARLEN) kend = min(kend, len);
    if (VARLEN && q0 >= len) kend = 0;  // every row is padding: no key tile to walk
    const int n_kt = (kend + kTile - 1) / kTile;
    int kend_w = CAUSAL ? qw + 32 : T;
    if (VARLEN) kend_w = min(kend_w, len);
    const bool wave_live = wave_rows && qw < row_limit;
    const int n_kt_w = wave_live ? min((kend_w + kTile - 1) / kTile, n_kt) : 0;  // tiles this wave uses

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
    // m: the exponents' maximum; neg_m = -m, or 0 while m = -inf.
    float m = kNegInf, neg_m = 0.0f, lsum = 0.0f;
    // O's move to a new maximum is applied one step late, just before the
    // next tile's products are added: the step that raises the maximum still
    // has the previous tile's products in flight.
    bool rescale = false;
    float alpha = 1.0f;
    auto apply_rescale = [&]() {
        if (rescale) {
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                oacc0[r] *= alpha;
                oacc1[r] *= alpha;
            }
        }
    };

    // Staging: 512 16-byte chunks per 64x64 tile; thread tid moves chunks
    // (row_a, col8) and (row_a + 32, col8) of a K tile and of a V^T tile.
    // They are buffer loads over the (batch, kv head) slice: the thread's
    // part of each address is a fixed register offset and the tile's part a
    // scalar one, so the loop spends no vector instructions on addresses.
    const int row_a = tid >> 3, row_b = row_a + 32, col8 = (tid & 7) * 8;
    const int slice_bytes = T * kHeadDim * 2;
    const __amdgpu_buffer_rsrc_t k_rsrc =
        __builtin_amdgcn_make_buffer_rsrc((void*)Kp, (short)0, slice_bytes, kBufferRsrcWord3);
    const __amdgpu_buffer_rsrc_t v_rsrc =
        __builtin_amdgcn_make_buffer_rsrc((void*)Vp, (short)0, slice_bytes, kBufferRsrcWord3);
    const int k_off_a = (row_a * kHeadDim + col8) * 2, k_off_b = (row_b * kHeadDim + col8) * 2;
    const int v_off_a = VROWS ? k_off_a : (row_a * T + col8) * 2;
    const int v_off_b = VROWS ? k_off_b : (row_b * T + col8) * 2;
    auto load_k = [&](int j, uint4& ra, uint4& rb) {
        const int tile = j * kTile * kHeadDim * 2;
        ra = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(k_rsrc, k_off_a, tile, 0));
        rb = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(k_rsrc, k_off_b, tile, 0));
    };
    auto load_v = [&](int j, uint4& ra, uint4& rb) {
        const int tile = VROWS ? j * kTile * kHeadDim * 2 : j * kTile * 2;
        ra = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(v_rsrc, v_off_a, tile, 0));
        rb = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(v_rsrc, v_off_b, tile, 0));
    };
    auto store_k = [&](int buf, const uint4& ra, const uint4& rb) {
        *(uint4*)&kls[buf][row_a * kLdsRow + col8] = ra;
        *(uint4*)&kls[buf][row_b * kLdsRow + col8] = rb;
    };
    auto store_v = [&](int j, int buf, uint4 ra, uint4 rb) {
        if (VROWS) {
            // rows are keys: keys at or past the length carry P = 0, so
            // their V rows are cleared (the padding may hold anything)
            if (VARLEN && j * kTile + row_a >= len) ra = make_uint4(0, 0, 0, 0);
            if (VARLEN && j * kTile + row_b >= len) rb = make_uint4(0, 0, 0, 0);
            *(uint4*)&vls[buf][vr_off(row_a, col8)] = ra;
            *(uint4*)&vls[buf][vr_off(row_b, col8)] = rb;
            return;
        }
        if (VARLEN && j * kTile + col8 + 8 > len) {
            // keys at or past the length carry P = 0: clear their V entries
            ra = clear_tail(ra, len - (j * kTile + col8));
            rb = clear_tail(rb, len - (j * kTile + col8));
        }
        // 68-half rows are 8-byte aligned: two 8-byte stores per chunk
        half_t* da = &vls[buf][row_a * kVRow + col8];
        half_t* db = &vls[buf][row_b * kVRow + col8];
        *(uint2*)da = make_uint2(ra.x, ra.y);
        *(uint2*)(da + 4) = make_uint2(ra.z, ra.w);
        *(uint2*)db = make_uint2(rb.x, rb.y);
        *(uint2*)(db + 4) = make_uint2(rb.z, rb.w);
    };
    // S^T = K Q^T for a tile's two 32-key blocks.
    auto scores = [&](const half_t* Ks, f32x16& s0, f32x16& s1) {
        s0 = zero16();
        s1 = zero16();
#pragma unroll
        for (int s = 0; s < 4; ++s) {
            const half8 a0 = *(const half8*)(Ks + l32 * kLdsRow + 16 * s + 8 * hi);
            const half8 a1 = *(const half8*)(Ks + (32 + l32) * kLdsRow + 16 * s + 8 * hi);
            s0 = mfma32(a0, qf[s], s0);
            s1 = mfma32(a1, qf[s], s1);
        }
    };
    // O^T += V^T P^T for one tile, P^T given as the 16 packed words of the
    // four 16-key k-steps.  k-step s covers the tile's keys 16 s + 4 hi + 0..3
    // and 16 s + 8 + 4 hi + 0..3 (the score accumulator's order), and V^T's A
    // operand is read in that same order.
    // Lane offsets of the transposed V row reads at k-step 0: rows
    // 4 hi + (lane % 16) / 4 and 8 more, columns d 0..31 then 32..63.
    int vr_tr[4];
    {
        const int r = 4 * hi + ((lane & 15) >> 2), cl = 16 * ((lane >> 4) & 1) + 4 * (lane & 3);
        vr_tr[0] = vr_off(r, cl);
        vr_tr[1] = vr_off(r + 8, cl);
        vr_tr[2] = vr_off(r, 32 + cl);
        vr_tr[3] = vr_off(r + 8, 32 + cl);
    }
    // VROWS: the same values come from the V row tile by transposed reads,
    // lane (d, hi) getting keys 16 s + 4 hi + 0..3 (then + 8) of column d.
    auto pv = [&](const half_t* Vs, const uint32_t (&w)[16]) {
#pragma unroll
        for (int s = 0; s < 4; ++s) {
            const half8 pb = half8_from_words(w[4 * s], w[4 * s + 1], w[4 * s + 2], w[4 * s + 3]);
            if (VROWS) {
                // rows 16 s + 4 hi + (lane % 16) / 4 (+ 8): 16 rows on keeps
                // the chunk key, so only the k-step moves the base
                const half_t* vs = Vs + 16 * s * kHeadDim;
                oacc0 = mfma32(cat(lds_read_tr(vs + vr_tr[0]), lds_read_tr(vs + vr_tr[1])), pb, oacc0);
                oacc1 = mfma32(cat(lds_read_tr(vs + vr_tr[2]), lds_read_tr(vs + vr_tr[3])), pb, oacc1);
            } else {
                const half_t* v0 = Vs + l32 * kVRow + 16 * s + 4 * hi;
                const half_t* v1 = v0 + 32 * kVRow;
                oacc0 = mfma32(cat(*(const half4*)v0, *(const half4*)(v0 + 8)), pb, oacc0);
                oacc1 = mfma32(cat(*(const half4*)v1, *(const half4*)(v1 + 8)), pb, oacc1);
            }
        }
    };

    // P = 2^(S c + nm) for a tile's 32 scores of this lane's query (nm is
    // minus the exponents' maximum), packed as binary16 pairs in accumulator
    // order; returns the lane's binary32 sum of the unrounded P.
    auto exponentials = [&](const f32x16& s0, const f32x16& s1, float nm, uint32_t (&p)[16]) {
        float sum = 0.0f;
#pragma unroll
        for (int r = 0; r < 16; r += 2) {
            const float p0 = exp2_fast(__builtin_fmaf(s0[r], c, nm));
            const float p1 = exp2_fast(__builtin_fmaf(s0[r + 1], c, nm));
            const float p2 = exp2_fast(__builtin_fmaf(s1[r], c, nm));
            const float p3 = exp2_fast(__builtin_fmaf(s1[r + 1], c, nm));
            sum += (p0 + p1) + (p2 + p3);
            p[r >> 1] = pack_half2(p0, p1);
            p[8 + (r >> 1)] = pack_half2(p2, p3);
        }
        return sum;
    };

    // One key tile j.  cur holds tile j's scores; the step forms tile j + 1's
    // scores into nxt and adds tile j - 1's products (P in pprev) to O while
    // it turns cur into P (pcur), then restages and synchronises.
    auto step = [&](int j, f32x16& cur0, f32x16& cur1, f32x16& nxt0, f32x16& nxt1,
                    const uint32_t (&pprev)[16], uint32_t (&pcur)[16]) {
        // Global loads in flight during this tile: K_{j+2} and V_{j+1}.
        const bool more_k = j + 2 < n_kt, more_v = j + 1 < n_kt;
        uint4 ka, kb, va, vb;
        if (more_k) load_k(j + 2, ka, kb);
        if (more_v) load_v(j + 1, va, vb);

        if (j < n_kt_w) {
            apply_rescale();
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
                    cur0[r] = m0 ? kNegInf : cur0[r];
                    cur1[r] = m1 ? kNegInf : cur1[r];
                }
            }

            // Matrix-core work of this step.  Tile j + 1's scores come from
            // the other K buffer; after the wave's last tile they are formed
            // from whatever it holds and never used.  At j = 0 there is no
            // previous tile: pprev is zero and V^T tile 0 stands in.
            // Raised wave priority over the interleaved stretch: of the two
            // waves on a SIMD, the one with matrix work in hand issues first.
            __builtin_amdgcn_s_setprio(1);
            scores(kls[(j + 1) & 1], nxt0, nxt1);
            pv(vls[j == 0 ? 0 : (j + 2) % 3], pprev);

            // P = 2^(S c - m) with the exponents' current maximum, the lane's
            // partial sum, and P^T packed as the B operand of the four 16-key
            // k-steps.
            float psum = exponentials(cur0, cur1, neg_m, pcur);
            SA_FWD_INTERLEAVE();
            __builtin_amdgcn_s_setprio(0);
            // The maximum moves (for every row of the wave, each to its own
            // running maximum) on the wave's first tile, which sets it, and
            // when some P may exceed 2^8; P is then formed again.  After the
            // first tile a row still at m = -inf has no admitted key at all
            // (key 0 is admitted to every query below the length), so its P
            // stay 0.  (The first-tile test sits inside the ballot: as a
            // separate || it lets the compiler sink the exponentials above
            // below the branch on steps where j may be 0, out of the
            // interleaved stretch.)
            if (__builtin_amdgcn_ballot_w64((psum > kMaxSum) | (j == 0)) != 0) {
                // Row maximum of the raw scores (c > 0, so max(S) c = max(S c)).
                float mx = fmaxf(cur0[0], cur1[0]);
#pragma unroll
                for (int r = 1; r < 16; ++r) mx = fmaxf(fmaxf(mx, cur0[r]), cur1[r]);
                const float m_new = fmaxf(m, max_halves(mx) * c);
                const float m_use = (m_new == kNegInf) ? 0.0f : m_new;
                psum = exponentials(cur0, cur1, -m_use, pcur);
                // l moves to the new maximum now, O (which still lacks tile
                // j - 1's products) at the start of the next step.
                alpha = exp2_fast(m - m_use);
                rescale = true;
                lsum = __builtin_fmaf(lsum, alpha, psum);
                m = m_new;
                neg_m = -m_use;
            } else {
                rescale = false;
                lsum += psum;
            }
        }

        // K_{j+2} replaces K_j (last read in the previous step) and V_{j+1}
        // replaces V_{j-2} (last read in the previous step).
        if (more_k) store_k(j & 1, ka, kb);
        if (more_v) store_v(j + 1, (j + 1) % 3, va, vb);
        vm_wait_all();  // nothing is outstanding here; keeps the compiler's count exact
        __syncthreads();
    };

    // Prologue: K_0, V_0, K_1 staged; tile 0's scores formed.
    {
        uint4 ka, kb, va, vb;
        if (n_kt > 0) {
            load_k(0, ka, kb);
            load_v(0, va, vb);
            store_k(0, ka, kb);
            store_v(0, 0, va, vb);
            if (n_kt > 1) {
                load_k(1, ka, kb);
                store_k(1, ka, kb);
            }
        }
    }
    __syncthreads();
    // Every global load issued so far (Q, the staged tiles) has landed: say so
    // to the compiler, which otherwise carries them as possibly outstanding
    // into the loop and waits on the loop's own prefetches before each tile.
    vm_wait_all();

    // Two register sets alternate roles from tile to tile, so nothing is copied.
    f32x16 sa0, sa1, sb0, sb1;
    uint32_t pa[16], pb[16];
#pragma unroll
    for (int i = 0; i < 16; ++i) pb[i] = 0u;
    if (n_kt_w > 0) scores(kls[0], sa0, sa1);
    for (int j = 0; j < n_kt; j += 2) {
        step(j, sa0, sa1, sb0, sb1, pb, pa);
        if (j + 1 < n_kt) step(j + 1, sb0, sb1, sa0, sa1, pa, pb);
    }
    // The wave's last tile's products (its V^T buffer is not restaged after it).
    if (n_kt_w > 0) {
        const int jl = n_kt_w - 1;
        apply_rescale();
        if (jl & 1) pv(vls[jl % 3], pb);
        else pv(vls[jl % 3], pa);
    }

    if (wave_rows) {
    // Epilogue: l over both halves, O / l, L = m + log2 l; rows with no
    // admitted key (l = 0) get O = 0 and L = -inf.  O goes through this
    // wave's own LDS rows so that the stores are whole 128-byte rows.
    const float l_tot = sum_halves(lsum);
    const bool empty = !(l_tot > 0.0f);
    const float inv = empty ? 0.0f : rcp_fast(l_tot);
    half_t* ow = &kls[0][0] + wave * 32 * kLdsRow;  // 32 rows x 72 halves per wave (kls is 2 x 64 rows)
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
    }  // wave_rows
    };
    process(items[0]);
    if (n_items == 2) {
        __syncthreads();  // the first item's epilogue staged O in kls
        process(items[1]);
    }
}

}  // namespace

int forward_order(const Shape& sh) {
    return tile_schedule(sh, (size_t)sh.batch * sh.heads, (sh.T + kFwdRows - 1) / kFwdRows);
}
size_t forward_blocks(const Shape& sh) {
    return tile_schedule_blocks(forward_order(sh), (size_t)sh.batch * sh.heads, (sh.T + kFwdRows - 1) / kFwdRows);
}

hipError_t launch_forward(const Shape& sh, const void* Q, const void* K, const void* Vt, void* O, float* L,
                          float c, hipStream_t stream) {
    const int n_qtiles = (sh.T + kFwdRows - 1) / kFwdRows;
    const int BH = sh.batch * sh.heads;
    dim3 grid((unsigned)forward_blocks(sh)), block(kFwdThreads);
    auto args = [&](auto kern) {
        hipLaunchKernelGGL(kern, grid, block, 0, stream, (const half_t*)Q, (const half_t*)K, (const half_t*)Vt,
                           (half_t*)O, L, sh.seqlens, c, sh.T, sh.heads, sh.kv_heads, n_qtiles, BH,
                           forward_order(sh));
    };
    const bool varlen = sh.seqlens != nullptr;
    auto go = [&](auto rows_tag) {
        constexpr bool R = decltype(rows_tag)::value;
        if (sh.causal) {
            if (varlen) args(sa_forward_kernel<true, true, R>);
            else args(sa_forward_kernel<true, false, R>);
        } else {
            if (varlen) args(sa_forward_kernel<false, true, R>);
            else args(sa_forward_kernel<false, false, R>);
        }
    };
    if (sh.v_rows) go(std::true_type{});
    else go(std::false_type{});
    return hipGetLastError();
}

}  // namespace sa
