// sa_backward.hip -- the split backward pass on gfx950: row terms, key pass
// (dK, dV, dS store) and dQ pass.
//
// Method: StreamingAttentionSM86 page, banner "The backward pass,
// deterministic and in two launches (no atomics)": P = 2^(S c - L),
// dP = dO V^T, D = rowsum(dO * O), dS = P (dP - D), dQ = s dS K,
// dK = s dS^T Q, dV = P^T dO; and banner "The query pass split in two around
// the key pass": the row terms D before the key pass, the key pass storing
// the score gradients it forms anyway, and dQ from the stored dS after it,
// so S, P and dP are formed once.
//
// MI355X design: every dense product runs on v_mfma_f32_32x32x16_f16.  The
// transposed operands the pages read from separate K^T / Q^T / dO^T copies
// come instead from LDS with ds_read_b64_tr_b16.  The GQA group sum of dK and
// dV is folded into the key pass (one workgroup per K/V head and key tile,
// its query heads in parallel wave pairs, summed through LDS in a fixed
// order), so there are no atomics and no partial-gradient planes.
#include <type_traits>

#include "sa_device.h"
#include "sa_internal.h"

namespace sa {

namespace {

// ---------------------------------------------------------------------------
// Row terms: D[b][h][i] = sum_d dO[b][h][i][d] * O[b][i][h*64 + d] in binary32
// (each fp16 widened, fused multiply-adds), 0 on padded rows.  Eight lanes
// per row, 16 bytes each of dO and O, reduced by three lane exchanges.
// ---------------------------------------------------------------------------
constexpr int kRowThreads = 256;
constexpr int kRowsPerBlock = kRowThreads / 8;

template <bool VARLEN>
__global__ __launch_bounds__(kRowThreads) void sa_row_terms_kernel(const half_t* __restrict__ dO,
                                                                    const half_t* __restrict__ O,
                                                                    float* __restrict__ D,
                                                                    const int32_t* __restrict__ seqlens, int T,
                                                                    int H, long long rows) {
    const long long row = (long long)blockIdx.x * kRowsPerBlock + (threadIdx.x >> 3);
    const int part = threadIdx.x & 7;
    float acc = 0.0f;
    const bool in = row < rows;
    int i = 0, b = 0, h = 0;
    if (in) {
        i = (int)(row % T);
        h = (int)((row / T) % H);
        b = (int)(row / ((long long)T * H));
        half8 g = *(const half8*)(dO + (size_t)row * kHeadDim + 8 * part);
        half8 o = *(const half8*)(O + (((size_t)b * T + i) * H + h) * kHeadDim + 8 * part);
#pragma unroll
        for (int t = 0; t < 8; ++t) acc = __builtin_fmaf((float)g[t], (float)o[t], acc);
    }
    acc += __shfl_xor(acc, 1);
    acc += __shfl_xor(acc, 2);
    acc += __shfl_xor(acc, 4);
    if (in && part == 0) {
        const bool valid = !VARLEN || i < min(max(seqlens[b], 0), T);
        D[row] = valid ? acc : 0.0f;
    }
}

// ---------------------------------------------------------------------------
// Key pass.  One workgroup per (batch, K/V head, 64-key tile kt); 2 GW waves:
// wave pair `slot` takes query heads kv G + slot, + GW, ... of the group in
// turn, and within a pair each wave owns 32 of the tile's keys.  Each pair
// walks its head's 32-query sub-tiles from the last down to the diagonal one
// (the pages' order), staging Q, dO, L and D of the sub-tile in LDS
// (double-buffered).  Per sub-tile and wave:
//   S  = Q K^T  (A = Q rows, LDS; B = K^T, registers)
//   dP = dO V^T (A = dO rows, LDS; B = V^T, registers, transposed once)
//   P  = 2^(S c - L),  dS = P (dP - D)  -- in registers, lane = key
//   dS stored as fp16 (the words of dK's product) into its 64x64 tile
//   dV^T += dO^T P, dK^T += Q^T dS (A = dO^T / Q^T by transposed LDS
//   reads, in the permuted query order of P's / dS's accumulators).
// The pairs' dK and dV are then summed through LDS in slot order, dK scaled
// by s, and stored with coalesced 16-byte writes.
// ---------------------------------------------------------------------------
constexpr int kSubRows = 32;
constexpr int kSubHalves = kSubRows * kLdsRow;
constexpr int kSlotBufBytes = 2 * kSubHalves * 2 + 2 * kSubRows * 4;  // Q, dO, L, D
constexpr int kRedRow = 68;                                             // floats

template <int GW>
struct KeyLds {
    static constexpr int stage = GW * 2 * kSlotBufBytes;
    static constexpr int red = GW * 64 * kRedRow * 4;
    static constexpr int vt = 64 * kLdsRow * 2;
    static constexpr int bytes = stage > red ? (stage > vt ? stage : vt) : (red > vt ? red : vt);
};

template <bool CAUSAL, bool VARLEN, int GW>
__global__ __launch_bounds__(128 * GW, 1) void sa_key_kernel(
    const half_t* __restrict__ Q, const half_t* __restrict__ K, const half_t* __restrict__ Vt,
    const half_t* __restrict__ dO, const float* __restrict__ L, const float* __restrict__ D,
    half_t* __restrict__ dS, float* __restrict__ dK, float* __restrict__ dVt,
    const int32_t* __restrict__ seqlens, float c, float s, int T, int H, int KV, int nkt, int BKV,
    int block_order, long long tiles_per_head) {
    constexpr int kThreads = 128 * GW;
    __shared__ __attribute__((aligned(16))) char smem[KeyLds<GW>::bytes];

    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
    const int l32 = lane & 31, hi = lane >> 5;
    const int slot = wave >> 1, khalf = wave & 1, st = tid & 127;

    int kt, bkv;
    if (block_order == 0) {  // key tile 0 first: it walks every query
        kt = (int)(blockIdx.x / BKV);
        bkv = (int)(blockIdx.x % BKV);
    } else {
        kt = (int)(blockIdx.x % nkt);
        bkv = (int)(blockIdx.x / nkt);
    }
    const int b = bkv / KV, kv = bkv % KV, G = H / KV;
    const int len = VARLEN ? min(max(seqlens[b], 0), T) : T;
    const int kbase = kt * kTile + 32 * khalf;  // this wave's first key
    const int key = kbase + l32;                // this lane's key

    // Query sub-tiles walked: whole 64-row tiles that the dQ pass reads.
    const int qlimit = VARLEN ? ((len + kTile - 1) / kTile) * kTile : T;
    const int sub_hi = qlimit / kSubRows;
    const int sub_lo = CAUSAL ? 2 * kt : 0;
    const bool tile_live = !VARLEN || kt * kTile < len;
    const int n_sub = tile_live ? max(0, sub_hi - sub_lo) : 0;
    const int n_items = n_sub * (G / GW);

    const size_t kv_off = ((size_t)b * KV + kv) * (size_t)T * kHeadDim;

    // K^T as the B operand of S = Q K^T: lane (key, hi) holds K[key][16 s + 8 hi + 0..7].
    half8 kf[4];
    {
        const half_t* kp = K + kv_off + (size_t)key * kHeadDim + 8 * hi;
#pragma unroll
        for (int q4 = 0; q4 < 4; ++q4) kf[q4] = *(const half8*)(kp + 16 * q4);
    }
    // V^T as the B operand of dP = dO V^T: lane (key, hi) needs V^T[16 s + 8 hi + 0..7][key],
    // a column of the V^T tile: stage the tile once and read it transposed.
    half8 vf[4];
    {
        half_t* vt_lds = (half_t*)smem;
        for (int chunk = tid; chunk < 512; chunk += kThreads) {
            int row = chunk >> 3, col = (chunk & 7) * 8;
            *(uint4*)&vt_lds[row * kLdsRow + col] =
                *(const uint4*)(Vt + kv_off + (size_t)row * T + kt * kTile + col);
        }
        __syncthreads();
#pragma unroll
        for (int q4 = 0; q4 < 4; ++q4) {
            half4 lo = lds_read_tr(vt_lds + tr_offset(lane, 16 * q4, 16 * q4 + 8, 32 * khalf));
            half4 hi4 = lds_read_tr(vt_lds + tr_offset(lane, 16 * q4 + 4, 16 * q4 + 12, 32 * khalf));
            vf[q4] = cat(lo, hi4);
        }
        __syncthreads();
    }

    f32x16 dkacc[2] = {zero16(), zero16()}, dvacc[2] = {zero16(), zero16()};

    // Staging of one item (head iteration gi, sub-tile sub) by the slot's 128 threads.
    uint4 qreg[2], oreg[2], lreg;
    auto item_head = [&](int it) { return kv * G + (it / n_sub) * GW + slot; };
    auto item_sub = [&](int it) { return sub_hi - 1 - (it % n_sub); };
    auto load_item = [&](int it) {
        const int head = item_head(it), sub = item_sub(it);
        const size_t rowbase = (((size_t)b * H + head) * T + (size_t)sub * kSubRows);
#pragma unroll
        for (int u = 0; u < 2; ++u) {
            int chunk = st + 128 * u, row = chunk >> 3, col = (chunk & 7) * 8;
            qreg[u] = *(const uint4*)(Q + (rowbase + row) * kHeadDim + col);
            oreg[u] = *(const uint4*)(dO + (rowbase + row) * kHeadDim + col);
        }
        if (st < 16) {
            const float* src = (st < 8) ? L : D;
            lreg = *(const uint4*)(src + rowbase + 4 * (st & 7));
        }
    };
    auto store_item = [&](int it, int buf) {
        const int sub = item_sub(it);
        char* sb = smem + (slot * 2 + buf) * kSlotBufBytes;
        half_t* Qs = (half_t*)sb;
        half_t* dOs = Qs + kSubHalves;
        float* LDs = (float*)(dOs + kSubHalves);
#pragma unroll
        for (int u = 0; u < 2; ++u) {
            int chunk = st + 128 * u, row = chunk >> 3, col = (chunk & 7) * 8;
            uint4 qv = qreg[u], ov = oreg[u];
            if (VARLEN && sub * kSubRows + row >= len) {  // padded rows never reach dK or dV
                qv = make_uint4(0, 0, 0, 0);
                ov = make_uint4(0, 0, 0, 0);
            }
            *(uint4*)&Qs[row * kLdsRow + col] = qv;
            *(uint4*)&dOs[row * kLdsRow + col] = ov;
        }
        if (st < 16) {
            uint4 v = lreg;
            if (VARLEN) {
                int r0 = sub * kSubRows + 4 * (st & 7);
                unsigned* e = (unsigned*)&v;
#pragma unroll
                for (int t = 0; t < 4; ++t)
                    if (r0 + t >= len) e[t] = 0u;
            }
            *(uint4*)&LDs[(st < 8 ? 0 : kSubRows) + 4 * (st & 7)] = v;
        }
    };

    if (n_items > 0) {
        load_item(0);
        store_item(0, 0);
    }
    __syncthreads();

    for (int it = 0; it < n_items; ++it) {
        const int buf = it & 1;
        if (it + 1 < n_items) load_item(it + 1);

        const int head = item_head(it), sub = item_sub(it);
        const int qb = sub * kSubRows;
        const char* sb = smem + (slot * 2 + buf) * kSlotBufBytes;
        const half_t* Qs = (const half_t*)sb;
        const half_t* dOs = Qs + kSubHalves;
        const float* Ls = (const float*)(dOs + kSubHalves);
        const float* Ds = Ls + kSubRows;
        // This wave's 32x32 block of the 64x64 dS^T tile [key][query].
        const int qt = sub >> 1;
        const size_t tile = CAUSAL ? (size_t)qt * (qt + 1) / 2 + kt : (size_t)qt * (T / kTile) + kt;
        half_t* dsp = dS + (((size_t)b * H + head) * (size_t)tiles_per_head + tile) * (kTile * kTile) +
                      (size_t)(32 * khalf + l32) * kTile + 32 * (sub & 1) + 4 * hi;

        const bool all_masked = (CAUSAL && qb + kSubRows - 1 < kbase) ||
                                (VARLEN && (qb >= len || kbase >= len));
        if (all_masked) {
            const half4 z = {(half_t)0.0f, (half_t)0.0f, (half_t)0.0f, (half_t)0.0f};
#pragma unroll
            for (int rg = 0; rg < 4; ++rg) *(half4*)(dsp + 8 * rg) = z;
        } else {
            f32x16 sacc = zero16(), pacc = zero16();
#pragma unroll
            for (int q4 = 0; q4 < 4; ++q4) {
                half8 aq = *(const half8*)(Qs + l32 * kLdsRow + 16 * q4 + 8 * hi);
                sacc = mfma32(aq, kf[q4], sacc);
            }
#pragma unroll
            for (int q4 = 0; q4 < 4; ++q4) {
                half8 ao = *(const half8*)(dOs + l32 * kLdsRow + 16 * q4 + 8 * hi);
                pacc = mfma32(ao, vf[q4], pacc);
            }
            const bool need_mask = (CAUSAL && qb < kbase + 31) || (VARLEN && (qb + kSubRows > len || kbase + 32 > len));
            half8 pp[2], pds[2];
#pragma unroll
            for (int rg = 0; rg < 4; ++rg) {
                const f32x4 lv = *(const f32x4*)(Ls + 8 * rg + 4 * hi);
                const f32x4 dv = *(const f32x4*)(Ds + 8 * rg + 4 * hi);
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const int r = 4 * rg + e;
                    float p = exp2_fast(__builtin_fmaf(sacc[r], c, -lv[e]));
                    float g = p * (pacc[r] - dv[e]);
                    if (need_mask) {
                        const int q = qb + 8 * rg + 4 * hi + e;
                        const bool masked = (CAUSAL && key > q) || (VARLEN && (q >= len || key >= len));
                        p = masked ? 0.0f : p;
                        g = masked ? 0.0f : g;
                    }
                    pp[r >> 3][r & 7] = to_half(p);
                    pds[r >> 3][r & 7] = to_half(g);
                }
            }
#pragma unroll
            for (int rg = 0; rg < 4; ++rg) {
                half4 v;
#pragma unroll
                for (int e = 0; e < 4; ++e) v[e] = pds[rg >> 1][4 * (rg & 1) + e];
                *(half4*)(dsp + 8 * rg) = v;
            }
            // dV^T += dO^T P and dK^T += Q^T dS; k-step ks covers queries
            // 16 ks + 4 hi + 0..3 and 16 ks + 8 + 4 hi + 0..3.
#pragma unroll
            for (int ks = 0; ks < 2; ++ks) {
#pragma unroll
                for (int db = 0; db < 2; ++db) {
                    half8 ao = cat(lds_read_tr(dOs + tr_offset(lane, 16 * ks, 16 * ks + 4, 32 * db)),
                                   lds_read_tr(dOs + tr_offset(lane, 16 * ks + 8, 16 * ks + 12, 32 * db)));
                    dvacc[db] = mfma32(ao, pp[ks], dvacc[db]);
                    half8 aq = cat(lds_read_tr(Qs + tr_offset(lane, 16 * ks, 16 * ks + 4, 32 * db)),
                                   lds_read_tr(Qs + tr_offset(lane, 16 * ks + 8, 16 * ks + 12, 32 * db)));
                    dkacc[db] = mfma32(aq, pds[ks], dkacc[db]);
                }
            }
        }

        if (it + 1 < n_items) store_item(it + 1, buf ^ 1);
        __syncthreads();
    }

    // Group sum through LDS in slot order, then coalesced stores.
    float* red = (float*)smem;
    const size_t key_row0 = ((size_t)b * KV + kv) * T + (size_t)kt * kTile;
    auto to_lds = [&](const f32x16& a0, const f32x16& a1) {
#pragma unroll
        for (int rg = 0; rg < 4; ++rg) {
            f32x4 v0 = {a0[4 * rg], a0[4 * rg + 1], a0[4 * rg + 2], a0[4 * rg + 3]};
            f32x4 v1 = {a1[4 * rg], a1[4 * rg + 1], a1[4 * rg + 2], a1[4 * rg + 3]};
            float* row = &red[(slot * 64 + 32 * khalf + l32) * kRedRow + 8 * rg + 4 * hi];
            *(f32x4*)row = v0;
            *(f32x4*)(row + 32) = v1;
        }
    };
    to_lds(dkacc[0], dkacc[1]);
    __syncthreads();
    for (int idx = tid; idx < 64 * 16; idx += kThreads) {  // dK[key][d]: 16 float4s per key
        const int kk = idx >> 4, d4 = (idx & 15) * 4;
        f32x4 v = *(const f32x4*)&red[kk * kRedRow + d4];
#pragma unroll
        for (int g = 1; g < GW; ++g) v += *(const f32x4*)&red[(g * 64 + kk) * kRedRow + d4];
        v *= s;
        *(f32x4*)(dK + (key_row0 + kk) * kHeadDim + d4) = v;
    }
    __syncthreads();
    to_lds(dvacc[0], dvacc[1]);
    __syncthreads();
    for (int idx = tid; idx < 64 * 16; idx += kThreads) {  // dV^T[d][key]: 16 float4s per d row
        const int d = idx >> 4, k4 = (idx & 15) * 4;
        f32x4 v;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            float a = red[(k4 + e) * kRedRow + d];
#pragma unroll
            for (int g = 1; g < GW; ++g) a += red[(g * 64 + k4 + e) * kRedRow + d];
            v[e] = a;
        }
        *(f32x4*)(dVt + (((size_t)b * KV + kv) * kHeadDim + d) * T + (size_t)kt * kTile + k4) = v;
    }
}

// ---------------------------------------------------------------------------
// dQ pass.  One 256-thread workgroup per 128 queries of a query head (two dS
// tile rows); wave w owns 32 queries.  For each key tile up to the diagonal
// (the query pass's order), the K tile and the block's two dS^T tiles are
// staged in LDS (double-buffered) and each wave accumulates
//   dQ^T += K^T dS^T   (A = K^T, B = dS^T, both by transposed LDS reads),
// so each lane ends with 4-float runs of one query's dQ row: dQ = s * sum,
// stored with 16-byte writes.
// ---------------------------------------------------------------------------
constexpr int kDqWaves = 4;
constexpr int kDqRows = 32 * kDqWaves;
constexpr int kDqThreads = 64 * kDqWaves;
constexpr int kTileHalvesDq = kTile * kLdsRow;

template <bool CAUSAL, bool VARLEN>
__global__ __launch_bounds__(kDqThreads, 2) void sa_dq_kernel(const half_t* __restrict__ K,
                                                               const half_t* __restrict__ dS,
                                                               float* __restrict__ dQ,
                                                               const int32_t* __restrict__ seqlens, float s,
                                                               int T, int H, int KV, int n_qblk, int BH,
                                                               int block_order, long long tiles_per_head) {
    __shared__ __attribute__((aligned(16))) half_t lds[2][3][kTileHalvesDq];  // [buf][K | dS row 0 | dS row 1]

    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
    const int l32 = lane & 31, hi = lane >> 5;
    int qblk, bh;
    if (block_order == 0) {
        qblk = n_qblk - 1 - (int)(blockIdx.x / BH);
        bh = (int)(blockIdx.x % BH);
    } else {
        qblk = (int)(blockIdx.x % n_qblk);
        bh = (int)(blockIdx.x / n_qblk);
    }
    const int b = bh / H, h = bh % H, kv = h / (H / KV);
    const int nt = T / kTile;
    const int len = VARLEN ? min(max(seqlens[b], 0), T) : T;
    const int ntl = VARLEN ? (len + kTile - 1) / kTile : nt;  // dS tile rows/cols in use
    const int qt0 = 2 * qblk;
    const int qt_w = qt0 + (wave >> 1);
    const int q = qblk * kDqRows + 32 * wave + l32;
    const bool wave_rows = qt_w < nt;

    int kt_end = CAUSAL ? min(qt0 + 2, nt) : nt;
    if (VARLEN) kt_end = min(kt_end, ntl);
    if (VARLEN && qt0 >= ntl) kt_end = 0;

    const half_t* Kp = K + ((size_t)b * KV + kv) * (size_t)T * kHeadDim;
    const half_t* dSh = dS + ((size_t)b * H + h) * (size_t)tiles_per_head * (kTile * kTile);
    auto tile_valid = [&](int qt, int kt) {
        return qt < nt && qt < ntl && (!CAUSAL || kt <= qt);
    };
    auto tile_ptr = [&](int qt, int kt) {
        size_t t = CAUSAL ? (size_t)qt * (qt + 1) / 2 + kt : (size_t)qt * nt + kt;
        return dSh + t * (kTile * kTile);
    };

    uint4 reg[6];
    auto load_tile = [&](int kt) {
#pragma unroll
        for (int u = 0; u < 2; ++u) {
            int chunk = tid + kDqThreads * u, row = chunk >> 3, col = (chunk & 7) * 8;
            reg[u] = *(const uint4*)(Kp + (size_t)(kt * kTile + row) * kHeadDim + col);
        }
#pragma unroll
        for (int r = 0; r < 2; ++r) {
            if (tile_valid(qt0 + r, kt)) {
                const half_t* tp = tile_ptr(qt0 + r, kt);
#pragma unroll
                for (int u = 0; u < 2; ++u) {
                    int chunk = tid + kDqThreads * u;
                    reg[2 + 2 * r + u] = *(const uint4*)(tp + chunk * 8);
                }
            }
        }
    };
    auto store_tile = [&](int kt, int buf) {
#pragma unroll
        for (int u = 0; u < 2; ++u) {
            int chunk = tid + kDqThreads * u, row = chunk >> 3, col = (chunk & 7) * 8;
            uint4 v = reg[u];
            if (VARLEN && kt * kTile + row >= len) v = make_uint4(0, 0, 0, 0);  // padded keys
            *(uint4*)&lds[buf][0][row * kLdsRow + col] = v;
        }
#pragma unroll
        for (int r = 0; r < 2; ++r) {
            if (tile_valid(qt0 + r, kt)) {
#pragma unroll
                for (int u = 0; u < 2; ++u) {
                    int chunk = tid + kDqThreads * u, row = chunk >> 3, col = (chunk & 7) * 8;
                    *(uint4*)&lds[buf][1 + r][row * kLdsRow + col] = reg[2 + 2 * r + u];
                }
            }
        }
    };

    f32x16 acc[2] = {zero16(), zero16()};
    if (kt_end > 0) {
        load_tile(0);
        store_tile(0, 0);
    }
    __syncthreads();
    for (int kt = 0; kt < kt_end; ++kt) {
        const int buf = kt & 1;
        if (kt + 1 < kt_end) load_tile(kt + 1);
        if (wave_rows && tile_valid(qt_w, kt)) {
            const half_t* Ks = lds[buf][0];
            const half_t* Ss = lds[buf][1 + (wave >> 1)];
            const int qcol = 32 * (wave & 1);
#pragma unroll
            for (int s4 = 0; s4 < 4; ++s4) {
                half8 bop = cat(lds_read_tr(Ss + tr_offset(lane, 16 * s4, 16 * s4 + 8, qcol)),
                                lds_read_tr(Ss + tr_offset(lane, 16 * s4 + 4, 16 * s4 + 12, qcol)));
#pragma unroll
                for (int db = 0; db < 2; ++db) {
                    half8 a = cat(lds_read_tr(Ks + tr_offset(lane, 16 * s4, 16 * s4 + 8, 32 * db)),
                                  lds_read_tr(Ks + tr_offset(lane, 16 * s4 + 4, 16 * s4 + 12, 32 * db)));
                    acc[db] = mfma32(a, bop, acc[db]);
                }
            }
        }
        if (kt + 1 < kt_end) store_tile(kt + 1, buf ^ 1);
        __syncthreads();
    }
    if (!wave_rows) return;
    float* dq = dQ + (((size_t)b * H + h) * T + q) * kHeadDim;
    const bool valid = !VARLEN || q < len;
#pragma unroll
    for (int db = 0; db < 2; ++db)
#pragma unroll
        for (int rg = 0; rg < 4; ++rg) {
            f32x4 v = {acc[db][4 * rg], acc[db][4 * rg + 1], acc[db][4 * rg + 2], acc[db][4 * rg + 3]};
            v *= valid ? s : 0.0f;
            *(f32x4*)(dq + 32 * db + 8 * rg + 4 * hi) = v;
        }
}

template <bool CAUSAL, bool VARLEN>
void launch_key_gw(int GW, dim3 grid, hipStream_t stream, const half_t* Q, const half_t* K, const half_t* Vt,
                   const half_t* dO, const float* L, const float* D, half_t* dS, float* dK, float* dVt,
                   const int32_t* seqlens, float c, float s, int T, int H, int KV, int nkt, int BKV, int order,
                   long long tph) {
#define SA_KEY_LAUNCH(gw)                                                                                    \
    hipLaunchKernelGGL((sa_key_kernel<CAUSAL, VARLEN, gw>), grid, dim3(128 * gw), 0, stream, Q, K, Vt, dO, L, \
                       D, dS, dK, dVt, seqlens, c, s, T, H, KV, nkt, BKV, order, tph)
    switch (GW) {
        case 4: SA_KEY_LAUNCH(4); break;
        case 3: SA_KEY_LAUNCH(3); break;
        case 2: SA_KEY_LAUNCH(2); break;
        default: SA_KEY_LAUNCH(1); break;
    }
#undef SA_KEY_LAUNCH
}

// Wave pairs per key-pass workgroup: the largest divisor of the group size
// that is at most 4.
int key_gw(int G) {
    for (int gw = 4; gw > 1; --gw)
        if (G % gw == 0) return gw;
    return 1;
}

}  // namespace

size_t row_terms_blocks(const Shape& sh) {
    size_t rows = (size_t)sh.batch * sh.heads * sh.T;
    return (rows + kRowsPerBlock - 1) / kRowsPerBlock;
}
size_t key_pass_blocks(const Shape& sh) { return (size_t)sh.batch * sh.kv_heads * (sh.T / kTile); }
size_t dq_pass_blocks(const Shape& sh) {
    return (size_t)sh.batch * sh.heads * ((sh.T + kDqRows - 1) / kDqRows);
}

hipError_t launch_row_terms(const Shape& sh, const void* dO, const void* O, float* D, hipStream_t stream) {
    long long rows = (long long)sh.batch * sh.heads * sh.T;
    dim3 grid((unsigned)row_terms_blocks(sh)), block(kRowThreads);
    if (sh.seqlens)
        hipLaunchKernelGGL(sa_row_terms_kernel<true>, grid, block, 0, stream, (const half_t*)dO, (const half_t*)O,
                           D, sh.seqlens, sh.T, sh.heads, rows);
    else
        hipLaunchKernelGGL(sa_row_terms_kernel<false>, grid, block, 0, stream, (const half_t*)dO,
                           (const half_t*)O, D, sh.seqlens, sh.T, sh.heads, rows);
    return hipGetLastError();
}

hipError_t launch_key_pass(const Shape& sh, const void* Q, const void* K, const void* Vt, const void* dO,
                           const float* L, const float* D, void* dS, float c, float s, float* dK, float* dVt,
                           hipStream_t stream) {
    const int nkt = sh.T / kTile, BKV = sh.batch * sh.kv_heads;
    const int GW = key_gw(sh.heads / sh.kv_heads);
    dim3 grid((unsigned)key_pass_blocks(sh));
    const long long tph = (long long)ds_tiles_per_head(sh);
    auto go = [&](auto causal_tag, auto varlen_tag) {
        constexpr bool C = decltype(causal_tag)::value, V = decltype(varlen_tag)::value;
        launch_key_gw<C, V>(GW, grid, stream, (const half_t*)Q, (const half_t*)K, (const half_t*)Vt,
                            (const half_t*)dO, L, D, (half_t*)dS, dK, dVt, sh.seqlens, c, s, sh.T, sh.heads,
                            sh.kv_heads, nkt, BKV, sh.block_order, tph);
    };
    using T_ = std::true_type;
    using F_ = std::false_type;
    if (sh.causal) {
        if (sh.seqlens) go(T_{}, T_{}); else go(T_{}, F_{});
    } else {
        if (sh.seqlens) go(F_{}, T_{}); else go(F_{}, F_{});
    }
    return hipGetLastError();
}

hipError_t launch_dq_pass(const Shape& sh, const void* K, const void* dS, float s, float* dQ,
                          hipStream_t stream) {
    const int n_qblk = (sh.T + kDqRows - 1) / kDqRows, BH = sh.batch * sh.heads;
    dim3 grid((unsigned)dq_pass_blocks(sh)), block(kDqThreads);
    const long long tph = (long long)ds_tiles_per_head(sh);
    auto go = [&](auto kern) {
        hipLaunchKernelGGL(kern, grid, block, 0, stream, (const half_t*)K, (const half_t*)dS, dQ, sh.seqlens, s,
                           sh.T, sh.heads, sh.kv_heads, n_qblk, BH, sh.block_order, tph);
    };
    if (sh.causal) {
        if (sh.seqlens) go(sa_dq_kernel<true, true>); else go(sa_dq_kernel<true, false>);
    } else {
        if (sh.seqlens) go(sa_dq_kernel<false, true>); else go(sa_dq_kernel<false, false>);
    }
    return hipGetLastError();
}

}  // namespace sa
