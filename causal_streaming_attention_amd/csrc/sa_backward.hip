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
#include <algorithm>
#include <type_traits>

#include "sa_device.h"
#include "sa_internal.h"

namespace sa {

namespace {



// ---------------------------------------------------------------------------
// Row terms: D[b][h][i] = sum_d dO[b][h][i][d] * O[b][i][h*64 + d] in binary32
// (each fp16 widened, fused multiply-adds), 0 on padded rows (which read
// nothing).  A block takes 64 rows of one (batch, head) (T is a multiple of
// 64); eight lanes per row, 16 bytes each of dO and O, reduced by three lane
// exchanges; each thread takes two rows 32 apart, so that all four of its
// loads are in flight at once.
// ---------------------------------------------------------------------------
constexpr int kRowThreads = 256;
constexpr int kRowsPerBlock = 64;

template <bool VARLEN>
__global__ __launch_bounds__(kRowThreads) void sa_row_terms_kernel(const half_t* __restrict__ dO,
                                                                    const half_t* __restrict__ O,
                                                                    float* __restrict__ D,
                                                                    const int32_t* __restrict__ seqlens, int T,
                                                                    int H) {
    const int tiles = T / kRowsPerBlock;
    const int bh = (int)blockIdx.x / tiles, i0 = ((int)blockIdx.x % tiles) * kRowsPerBlock;
    const int b = bh / H, h = bh % H;
    const int part = threadIdx.x & 7, r = threadIdx.x >> 3;  // rows i0 + r and i0 + r + 32
    const size_t drow = (size_t)bh * T + i0 + r;
    const size_t orow = ((size_t)b * T + i0 + r) * H + h;
    // Rows at or past the length (padding) get D = 0 without reading dO or O.
    const int len = VARLEN ? min(max(seqlens[b], 0), T) : T;
    const bool in0 = !VARLEN || i0 + r < len, in1 = !VARLEN || i0 + r + 32 < len;
    half8 g0 = {}, g1 = {}, o0 = {}, o1 = {};
    if (in0) {
        g0 = *(const half8*)(dO + drow * kHeadDim + 8 * part);
        o0 = *(const half8*)(O + orow * kHeadDim + 8 * part);
    }
    if (in1) {
        g1 = *(const half8*)(dO + (drow + 32) * kHeadDim + 8 * part);
        o1 = *(const half8*)(O + (orow + 32 * (size_t)H) * kHeadDim + 8 * part);
    }
    float a0 = 0.0f, a1 = 0.0f;
#pragma unroll
    for (int t = 0; t < 8; ++t) {
        a0 = __builtin_fmaf((float)g0[t], (float)o0[t], a0);
        a1 = __builtin_fmaf((float)g1[t], (float)o1[t], a1);
    }
    a0 += __shfl_xor(a0, 1);
    a1 += __shfl_xor(a1, 1);
    a0 += __shfl_xor(a0, 2);
    a1 += __shfl_xor(a1, 2);
    a0 += __shfl_xor(a0, 4);
    a1 += __shfl_xor(a1, 4);
    if (part == 0) {
        D[drow] = in0 ? a0 : 0.0f;
        D[drow + 32] = in1 ? a1 : 0.0f;
    }
}

// ---------------------------------------------------------------------------
// Key pass.  One workgroup per (batch, K/V head, 64-key tile kt), or per pair
// of key tiles (p, nkt - 1 - p) taken one after the other; 2 GW waves:
// wave (slot, khalf) takes query heads kv G + slot, + GW, ... of the group in
// turn and owns keys kt * 64 + 32 khalf + 0..31.  (On grids too small for the
// chip, a group of one or two heads gets more slots than heads, GW = G R:
// slot s takes head s % G's sub-tiles sub_hi - 1 - s / G and every R-th
// below it, and the group sum adds the R phases like heads.)  Each wave
// walks its head's 32-query sub-tiles from the last down to the diagonal one
// (the pages' order) on its own: it stages each sub-tile's Q, dO, L and D into a private
// LDS double buffer with direct global-to-LDS loads, one sub-tile ahead, so
// the loop has no workgroup barrier and the waves sharing a SIMD drift apart
// and overlap their matrix and vector work.  Per sub-tile and wave:
//   S  = Q K^T  (A = Q rows, LDS; B = K^T, registers)
//   dP = dO V^T (A = dO rows, LDS; B = V^T, registers, transposed once)
//   P  = 2^(S c - L),  dS = P (dP - D)  -- in registers, lane = key
//   dS stored as fp16 (the words of dK's product) into its 64x64 tile
//   dV^T += dO^T P, dK^T += Q^T dS (A = dO^T / Q^T by transposed LDS
//   reads, in the permuted query order of P's / dS's accumulators).
// The dV / dK products of a sub-tile are issued one sub-tile late, spread
// through the next sub-tile's vector work at raised wave priority.  With V
// as rows (v_rows), V's operand is loaded straight from its rows and dV is
// written as rows.  The slots' dK and dV are then summed through LDS in slot
// order, dK scaled by s, and stored with coalesced 16-byte writes.
//
// A staged 32 x 64 fp16 sub-tile has 128-byte rows whose 16-byte chunks are
// permuted per row (swz below) so that its reads meet no bank conflict
// without padding (which direct loads cannot make).
// ---------------------------------------------------------------------------
constexpr int kSubRows = 32;
constexpr int kSubBytes = kSubRows * kHeadDim * 2;          // 4096
// Q, dO, then two 256-byte blocks: L in the first's lanes 0..31, D in the
// second's lanes 32..63 (each written by a 64-lane load whose other lanes
// fall outside its resource).
constexpr int kItemBytes = 2 * kSubBytes + 2 * 64 * 4;          // 8704
constexpr int kDOffsetFloats = 64 + 32;                          // D block, lane 32
constexpr int kWaveBytes = 2 * kItemBytes;
constexpr int kRedRow = 68;                                  // floats

template <int GW>
struct KeyLds {
    static constexpr int stage = 2 * GW * kWaveBytes;        // per wave: two items
    static constexpr int red = GW * 64 * kRedRow * 4;
    static constexpr int vt = 64 * kLdsRow * 2;
    static constexpr int bytes = stage > red ? (stage > vt ? stage : vt) : (red > vt ? red : vt);
};

// The chunk permutation of a staged sub-tile's row: LDS moves 256 bytes (64
// banks) a cycle, two 128-byte rows side by side, so a 16-byte row read by 16
// lanes (16 consecutive rows, one chunk) is free of bank conflicts when f(r)
// is distinct over the 8 rows of each parity among them: f takes bits 1..3 of
// r.  A transposed read covers 4 rows x 2 chunks of an aligned group of 4
// rows, in which the two rows of a parity must land in different 4-chunk
// halves: bit 2 of f(r) is bit 1 of r.
__device__ __forceinline__ int swz_key(int row) { return (((row >> 1) & 1) << 2) | ((row >> 2) & 3); }
// The dQ pass's K tiles are only read transposed: a key that depends on the
// row's low three bits suffices (rows r and r + 2 of an aligned group of 4 in
// different 4-chunk halves), and keeps that kernel's addressing cheap.
__device__ __forceinline__ int swz_key_k(int row) { return ((row & 3) << 1) | ((row >> 2) & 1); }
// Element offset of (row, col) in a swizzled 32 x 64 sub-tile.
__device__ __forceinline__ int swz(int row, int col) {
    return row * kHeadDim + (((col >> 3) ^ swz_key(row)) << 3) + (col & 7);
}

// Issue-order hint: a group of n instructions of one kind (0x008 matrix,
// 0x010 vector memory) at this point of the schedule.
#define SA_SGB(mask, n) __builtin_amdgcn_sched_group_barrier(mask, n, 0)

typedef __attribute__((address_space(3))) void lds_void;

__device__ __forceinline__ void dma16(const void* g, char* lds_wave_base) {
    __builtin_amdgcn_global_load_lds(g, (lds_void*)((__attribute__((address_space(3))) char*)lds_wave_base), 16, 0, 0);
}
// 16-byte buffer load at soffset + voffset + OFF within the resource into
// LDS at lds_wave_base + OFF + 16 lane (the offset field moves both
// addresses; the scalar offset only the memory address).
template <int OFF>
__device__ __forceinline__ void dma16_buf(__amdgpu_buffer_rsrc_t r, uint32_t voffset, uint32_t soffset,
                                          char* lds_wave_base) {
    __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_void*)((__attribute__((address_space(3))) char*)lds_wave_base),
                                             16, voffset, soffset, OFF, 0);
}
__device__ __forceinline__ void dma4_buf(__amdgpu_buffer_rsrc_t r, uint32_t voffset, char* lds_wave_base) {
    __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_void*)((__attribute__((address_space(3))) char*)lds_wave_base),
                                             4, voffset, 0, 0, 0);
}

template <bool CAUSAL, bool VARLEN, int GW>
__global__ __launch_bounds__(128 * GW, 2) void sa_key_kernel(
    const half_t* __restrict__ Q, const half_t* __restrict__ K, const half_t* __restrict__ Vt,
    const half_t* __restrict__ dO, const float* __restrict__ L, const float* __restrict__ D,
    half_t* __restrict__ dS, float* __restrict__ dK, float* __restrict__ dVt,
    const int32_t* __restrict__ seqlens, float c, float s, int T, int H, int KV, int nkt, int BKV,
    int block_order, Chunk ch, int v_rows, ProjectionOut kproj, ProjectionOut vproj) {
    constexpr int kThreads = 128 * GW;
    __shared__ __attribute__((aligned(16))) char smem[KeyLds<GW>::bytes];

    const int tid = threadIdx.x, wave = wave_id(), lane = tid & 63;
    const int l32 = lane & 31, hi = lane >> 5;
    const int slot = wave >> 1, khalf = wave & 1;
    const bool store_ds = dS != nullptr;

    int kt_first, kt_second = -1, bkv;
    if (VARLEN && block_order == 0 && BKV / KV <= kMaxRankedBatch) {
        // Variable lengths: the longest sequences' key tiles first (their
        // walks are the longest), key tile 0 first within each.
        const int per_b = KV * nkt;
        const int r = (int)blockIdx.x / per_b, rest = (int)blockIdx.x % per_b;
        kt_first = rest / KV;
        bkv = batch_of_rank(seqlens, BKV / KV, T, r) * KV + rest % KV;
    } else if (!VARLEN && block_order == kOrderKeyPairs) {
        // Key tiles p and nkt - 1 - p: every workgroup walks the same number
        // of sub-tiles (causal), so a grid that fits the chip at once ends
        // together instead of leaving a second round to the dispatcher.
        const int p = (int)(blockIdx.x / BKV);
        bkv = (int)(blockIdx.x % BKV);
        kt_first = p;
        if (nkt - 1 - p != p) kt_second = nkt - 1 - p;
    } else if (block_order == 0) {  // key tile 0 first: it walks every query
        kt_first = (int)(blockIdx.x / BKV);
        bkv = (int)(blockIdx.x % BKV);
    } else {
        kt_first = (int)(blockIdx.x % nkt);
        bkv = (int)(blockIdx.x / nkt);
    }
    auto process = [&](const int kt) {
    const int b = bkv / KV, kv = bkv % KV, G = H / KV;
    const int len = VARLEN ? min(max(seqlens[b], 0), T) : T;
    const int kbase = kt * kTile + 32 * khalf;  // this wave's first key
    const int key = kbase + l32;                // this lane's key

    // Query sub-tiles walked: whole 64-row tiles that the dQ pass reads, in
    // the chunk's query tiles [ch.q_lo, ch.q_hi).
    const int qlimit = VARLEN ? ((len + kTile - 1) / kTile) * kTile : T;
    const int sub_hi = min(qlimit / kSubRows, 2 * ch.q_hi);
    const int sub_lo = CAUSAL ? max(2 * kt, 2 * ch.q_lo) : 2 * ch.q_lo;
    const bool tile_live = !VARLEN || kt * kTile < len;
    const int n_sub = tile_live ? max(0, sub_hi - sub_lo) : 0;
    // Split walk when there are more slots than heads (GW = G R): this slot's
    // phase and its share of the sub-tiles.
    const bool split = GW > G;
    const int R = split ? GW / G : 1, phase = split ? slot / G : 0;
    const int n_items = split ? (n_sub > phase ? (n_sub - phase + R - 1) / R : 0) : n_sub * (G / GW);

    const size_t kv_off = ((size_t)b * KV + kv) * (size_t)T * kHeadDim;

    // The score and dP products' B operands, held for the whole walk.  A key
    // tile past the length (variable lengths) walks nothing and loads
    // neither: its dK and dV are the zeros the group sum below writes.
    // n_sub is the same for every wave of the workgroup, so the barriers
    // stay paired.
    half8 kf[4], vf[4];
    if (!VARLEN || n_sub > 0) {
        // K^T as the B operand of S = Q K^T: lane (key, hi) holds K[key][16 s + 8 hi + 0..7].
        {
            const half_t* kp = K + kv_off + (size_t)key * kHeadDim + 8 * hi;
#pragma unroll
            for (int q4 = 0; q4 < 4; ++q4) kf[q4] = *(const half8*)(kp + 16 * q4);
        }
        // V^T as the B operand of dP = dO V^T: lane (key, hi) needs V^T[16 s + 8 hi + 0..7][key],
        // a row of V when V comes as rows, else a column of the V^T tile: stage
        // that tile once and read it transposed.
        if (v_rows) {
            const half_t* vp = Vt + kv_off + (size_t)key * kHeadDim + 8 * hi;
#pragma unroll
            for (int q4 = 0; q4 < 4; ++q4) vf[q4] = *(const half8*)(vp + 16 * q4);
        } else {
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
    }

    f32x16 dkacc0 = zero16(), dkacc1 = zero16(), dvacc0 = zero16(), dvacc1 = zero16();

    char* const wstage = smem + wave * kWaveBytes;  // this wave's two item buffers
    const int dma_row = lane >> 3;                         // + 8 u
    // Direct loads of one item into buffer `buf`: 4 x 1 KB of Q rows, 4 x 1 KB
    // of dO rows (lane l of load u: row 8 u + l / 8, stored chunk l % 8 holding
    // the row's chunk (l % 8) ^ swz_key(row)), then L into the first 256-byte
    // block (lanes 0..31) and D into the second (lanes 32..63).
    // Row 16 u + r has the chunk permutation of row r, so loads u and u + 2
    // differ by 2 KB in memory and in LDS: the instruction's offset field.
    const uint32_t dma_off0 = (uint32_t)(dma_row * kHeadDim + ((lane & 7) ^ swz_key(dma_row)) * 8) * 2u;
    const uint32_t dma_off1 = (uint32_t)(dma_row * kHeadDim + ((lane & 7) ^ swz_key(dma_row + 8)) * 8) * 2u;
    // The item's rows as buffer resources built on the scalar unit: the loads
    // take fixed per-lane offsets, so no vector instruction forms an address.
    // Q and dO: one resource per head over its T rows (rebuilt only when the
    // walk moves on to the slot's next head), the sub-tile a scalar offset of
    // sub x 4 KB; the record count bounds the per-lane offsets to the head.
    // L's and D's resources hold the item's 32 values each; the other 32
    // lanes of their 64-lane loads fall outside and fill unused slots with
    // zeros.
    const uint32_t ld_off_l = 4u * (uint32_t)lane, ld_off_d = 4u * (uint32_t)lane - 128u;
    auto rows_rsrc = [&](const half_t* p, int hd) {
        return __builtin_amdgcn_make_buffer_rsrc((void*)(p + ((size_t)b * H + hd) * T * kHeadDim), (short)0,
                                                 T * kHeadDim * 2, kBufferRsrcWord3);
    };
    int dma_head = kv * G + slot;
    __amdgpu_buffer_rsrc_t q_head = rows_rsrc(Q, dma_head), o_head = rows_rsrc(dO, dma_head);
    const float* l_head = L + ((size_t)b * H + dma_head) * T;
    const float* d_head = D + ((size_t)b * H + dma_head) * T;
    auto issue_item = [&](int head, int sub, int buf) {
        if (head != dma_head) {
            dma_head = head;
            q_head = rows_rsrc(Q, head);
            o_head = rows_rsrc(dO, head);
            l_head = L + ((size_t)b * H + head) * T;
            d_head = D + ((size_t)b * H + head) * T;
        }
        const uint32_t so = (uint32_t)sub * (uint32_t)kSubBytes;
        char* base = wstage + buf * kItemBytes;
        dma16_buf<0>(q_head, dma_off0, so, base);
        dma16_buf<1024>(q_head, dma_off1, so, base);
        dma16_buf<2048>(q_head, dma_off0, so, base);
        dma16_buf<3072>(q_head, dma_off1, so, base);
        dma16_buf<0>(o_head, dma_off0, so, base + kSubBytes);
        dma16_buf<1024>(o_head, dma_off1, so, base + kSubBytes);
        dma16_buf<2048>(o_head, dma_off0, so, base + kSubBytes);
        dma16_buf<3072>(o_head, dma_off1, so, base + kSubBytes);
        const int r = sub * kSubRows;
        dma4_buf(__builtin_amdgcn_make_buffer_rsrc((void*)(l_head + r), (short)0, kSubRows * 4, kBufferRsrcWord3),
                 ld_off_l, base + 2 * kSubBytes);
        dma4_buf(__builtin_amdgcn_make_buffer_rsrc((void*)(d_head + r), (short)0, kSubRows * 4, kBufferRsrcWord3),
                 ld_off_d, base + 2 * kSubBytes + 256);
    };

    // The dS store's per-head base, rebuilt when the walk reaches the slot's next head.
    int ds_head_id = -1;
    half_t* ds_head = dS;
    // Items in order: for each of the slot's heads, sub-tiles from the last
    // down (every R-th from its phase on a split walk).
    int head = kv * G + (split ? slot % G : slot), sub = sub_hi - 1 - phase;
    if (n_items > 0) issue_item(head, sub, 0);
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");  // the first item has landed in LDS
    // ... and K's fragments: say so to the compiler too, which otherwise keeps
    // them as possibly outstanding and drains every load before the products.
    vm_wait_all();

    // Transposed reads of a staged item's dO^T and Q^T rows, the A operands of
    // its dV^T += dO^T P and dK^T += Q^T dS products; k-step ks covers queries
    // 16 ks + 4 hi + 0..3 and 16 ks + 8 + 4 hi + 0..3.  Transposed read: lane
    // l gets column (16 ((l / 16) % 2) + l % 16) of rows row0 + 0..3.
    // Row r + 16 has row r's chunk permutation, so of the 16 reads only the
    // rows r and r + 8 and the column halves (d 0..31 and 32..63) need their
    // own lane addresses; k-steps and Q versus dO are offsets of 2 and 4 KB.
    const int trr = (lane & 15) >> 2, trc = 16 * ((lane >> 4) & 1) + 4 * (lane & 3);
    const int tr_row = 4 * hi + trr;
    const uint32_t tr_a0 = (uint32_t)swz(tr_row, trc) * 2u, tr_a1 = (uint32_t)swz(tr_row, 32 + trc) * 2u;
    const uint32_t tr_b0 = (uint32_t)swz(tr_row + 8, trc) * 2u, tr_b1 = (uint32_t)swz(tr_row + 8, 32 + trc) * 2u;
    auto read_transposed = [&](const half_t* Qs, half4 (&t)[16]) {
        const uint32_t q = lds_addr(Qs);
        const uint32_t a0 = q + tr_a0, a1 = q + tr_a1, b0 = q + tr_b0, b1 = q + tr_b1;
        t[0] = lds_read_tr_at<kSubBytes>(a0);
        t[1] = lds_read_tr_at<kSubBytes>(b0);
        t[2] = lds_read_tr_at<kSubBytes>(a1);
        t[3] = lds_read_tr_at<kSubBytes>(b1);
        t[4] = lds_read_tr_at<0>(a0);
        t[5] = lds_read_tr_at<0>(b0);
        t[6] = lds_read_tr_at<0>(a1);
        t[7] = lds_read_tr_at<0>(b1);
        t[8] = lds_read_tr_at<kSubBytes + 2048>(a0);
        t[9] = lds_read_tr_at<kSubBytes + 2048>(b0);
        t[10] = lds_read_tr_at<kSubBytes + 2048>(a1);
        t[11] = lds_read_tr_at<kSubBytes + 2048>(b1);
        t[12] = lds_read_tr_at<2048>(a0);
        t[13] = lds_read_tr_at<2048>(b0);
        t[14] = lds_read_tr_at<2048>(a1);
        t[15] = lds_read_tr_at<2048>(b1);
        lds_wait(t[0], t[1], t[2], t[3], t[4], t[5], t[6], t[7]);
        lds_wait(t[8], t[9], t[10], t[11], t[12], t[13], t[14], t[15]);
    };
    auto accumulate = [&](const half4 (&t)[16], const uint32_t (&wp)[8], const uint32_t (&wd)[8]) {
        const half8 pp0 = half8_from_words(wp[0], wp[1], wp[2], wp[3]);
        const half8 pp1 = half8_from_words(wp[4], wp[5], wp[6], wp[7]);
        const half8 pd0 = half8_from_words(wd[0], wd[1], wd[2], wd[3]);
        const half8 pd1 = half8_from_words(wd[4], wd[5], wd[6], wd[7]);
        dvacc0 = mfma32(cat(t[0], t[1]), pp0, dvacc0);
        dvacc1 = mfma32(cat(t[2], t[3]), pp0, dvacc1);
        dkacc0 = mfma32(cat(t[4], t[5]), pd0, dkacc0);
        dkacc1 = mfma32(cat(t[6], t[7]), pd0, dkacc1);
        dvacc0 = mfma32(cat(t[8], t[9]), pp1, dvacc0);
        dvacc1 = mfma32(cat(t[10], t[11]), pp1, dvacc1);
        dkacc0 = mfma32(cat(t[12], t[13]), pd1, dkacc0);
        dkacc1 = mfma32(cat(t[14], t[15]), pd1, dkacc1);
    };

    // P and dS of the previous item, packed as binary16 pairs in accumulator
    // order: the B operands of its dV and dK products, which run inside this
    // item's vector work.  Before the first item they are zero and the first
    // item's own (finite) rows stand in for the previous item's, so those
    // products add exact zeros.
    uint32_t wp[8], wd[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) wp[i] = wd[i] = 0u;

    for (int it = 0; it < n_items; ++it) {
        const int buf = it & 1;
        // This item's loads were issued in the previous item, and only that
        // item's two dS stores (if dS is stored) are younger: wait for the
        // loads, not for the stores to reach memory.
        if (store_ds) asm volatile("s_waitcnt vmcnt(2)" ::: "memory");
        else asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
        int next_head = head, next_sub = sub - R;
        if (!split && next_sub < sub_lo) {
            next_sub = sub_hi - 1;
            next_head += GW;
        }
        const int qb = sub * kSubRows;
        half_t* Qs = (half_t*)(wstage + buf * kItemBytes);
        half_t* dOs = Qs + kSubRows * kHeadDim;
        float* Ls = (float*)(dOs + kSubRows * kHeadDim);
        float* Ds = Ls + kDOffsetFloats;
        if (VARLEN && qb + kSubRows > len) {
            // Rows at or past the length never reach dK or dV: clear them.
            const int keep = max(len - qb, 0);
#pragma unroll
            for (int u = 0; u < 4; ++u) {
                const int row = 8 * u + dma_row;
                if (row >= keep) {
                    *(uint4*)(Qs + row * kHeadDim + (lane & 7) * 8) = make_uint4(0, 0, 0, 0);
                    *(uint4*)(dOs + row * kHeadDim + (lane & 7) * 8) = make_uint4(0, 0, 0, 0);
                }
            }
            if ((lane & 31) >= keep) (lane < 32 ? Ls : Ds)[lane & 31] = 0.0f;
        }
        // This item's score and dP operands first, so that one wait covers
        // them and the previous item's transposed operands.
        half8 qa[4], da[4];
#pragma unroll
        for (int q4 = 0; q4 < 4; ++q4) {
            qa[q4] = *(const half8*)(Qs + swz(l32, 16 * q4 + 8 * hi));
            da[q4] = *(const half8*)(dOs + swz(l32, 16 * q4 + 8 * hi));
        }
        // The previous item's transposed operands; once they are in registers
        // its buffer takes the next item.
        half4 t[16];
        read_transposed((const half_t*)(wstage + (it == 0 ? buf : buf ^ 1) * kItemBytes), t);
        // Always issued (the last item loads its own rows again into the free
        // buffer), so that the loads share a block with the products below
        // and go out between them.  Raised wave priority from here to the end
        // of the item: of the two waves on a SIMD, the one past its operand
        // reads and waits (with matrix and vector work in hand) issues first.
        const bool more = it + 1 < n_items;
        __builtin_amdgcn_s_setprio(1);
        issue_item(more ? next_head : head, more ? next_sub : sub, buf ^ 1);

        // A block with no admitted pair (the diagonal sub-tile of the upper key
        // half, padding) goes through the same code: the mask makes its P and
        // dS exact zeros.
        f32x16 sacc = zero16(), pacc = zero16();
#pragma unroll
        for (int q4 = 0; q4 < 4; ++q4) sacc = mfma32(qa[q4], kf[q4], sacc);
#pragma unroll
        for (int q4 = 0; q4 < 4; ++q4) pacc = mfma32(da[q4], vf[q4], pacc);
        f32x4 lv[4], dv[4];
#pragma unroll
        for (int rg = 0; rg < 4; ++rg) {
            lv[rg] = *(const f32x4*)(Ls + 8 * rg + 4 * hi);
            dv[rg] = *(const f32x4*)(Ds + 8 * rg + 4 * hi);
        }
        // The next item's direct loads between this item's score and dP products.
        SA_SGB(0x008, 1); SA_SGB(0x010, 2); SA_SGB(0x008, 1); SA_SGB(0x010, 2);
        SA_SGB(0x008, 1); SA_SGB(0x010, 2); SA_SGB(0x008, 1); SA_SGB(0x010, 2);
        SA_SGB(0x008, 1); SA_SGB(0x010, 2); SA_SGB(0x008, 3);
        // The previous item's products go into the matrix pipe behind these;
        // the compiler's own schedule places them among this item's vector
        // instructions (a fixed one-product-per-eight pattern was slower).
        __builtin_amdgcn_sched_barrier(0);
        accumulate(t, wp, wd);
        float p[16], g[16];
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            p[r] = exp2_fast(__builtin_fmaf(sacc[r], c, -lv[r >> 2][r & 3]));
            g[r] = p[r] * (pacc[r] - dv[r >> 2][r & 3]);
        }
        const bool need_mask = (CAUSAL && qb < kbase + 31) || (VARLEN && (qb + kSubRows > len || kbase + 32 > len));
        if (need_mask) {
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int q = qb + 8 * (r >> 2) + 4 * hi + (r & 3);
                const bool masked = (CAUSAL && key > q) || (VARLEN && (q >= len || key >= len));
                p[r] = masked ? 0.0f : p[r];
                g[r] = masked ? 0.0f : g[r];
            }
        }
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            wp[i] = pack_half2(p[2 * i], p[2 * i + 1]);
            wd[i] = pack_half2(g[2 * i], g[2 * i + 1]);
        }
        // dS to the workspace (when there is one): this wave's 32x32 block of
        // the 64x64 tile is quadrant (query half sub % 2, key half khalf), and
        // each lane stores its key's 16 queries as the accumulator holds them
        // (two 16-byte words: its queries of rows 0..15, then of 16..31), so a
        // wave writes two fully coalesced 1 KB runs.  The dQ pass turns them
        // into its operand layout.  Non-temporal: dS is written once and read
        // once; streamed past L2 it neither evicts the Q/dO rows the walk
        // reuses nor stalls the walk behind L2 write-backs.
        if (store_ds) {
            if (head != ds_head_id) {
                ds_head_id = head;
                ds_head = dS + ((size_t)b * H + head) * (size_t)ch.tph * (kTile * kTile);
            }
            // Tile indices stay below 2^31 (T <= 2^20: at most 2^27 tiles per head).
            const uint32_t qt = (uint32_t)sub >> 1;
            const uint32_t tile = (CAUSAL ? (qt * (qt + 1)) >> 1 : qt * (uint32_t)(T / kTile)) + (uint32_t)kt -
                                  (uint32_t)ch.tile0;
            half_t* dsp = ds_head + (size_t)tile * (kTile * kTile) + (2 * (sub & 1) + khalf) * 1024 + 8 * lane;
            __builtin_nontemporal_store(half8_from_words(wd[0], wd[1], wd[2], wd[3]), (half8*)dsp);
            __builtin_nontemporal_store(half8_from_words(wd[4], wd[5], wd[6], wd[7]), (half8*)(dsp + 512));
        }
        __builtin_amdgcn_s_setprio(0);  // the next item's reads and waits at normal priority
        head = next_head;
        sub = next_sub;
    }
    // The last item's products.
    if (n_items > 0) {
        half4 t[16];
        read_transposed((const half_t*)(wstage + ((n_items - 1) & 1) * kItemBytes), t);
        accumulate(t, wp, wd);
    }
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();  // every wave is done with its staging buffers

    // Group sum through LDS in slot order, then coalesced stores: dK's and
    // dV's partials side by side (together they fill the staging space), so
    // one barrier covers both.
    float* red = (float*)smem;
    float* red_v = red + GW * 64 * kRedRow;
    static_assert(2 * KeyLds<GW>::red <= KeyLds<GW>::bytes, "dK and dV partials share the LDS");
    const size_t key_row0 = ((size_t)b * KV + kv) * T + (size_t)kt * kTile;
    auto to_lds = [&](float* dst, const f32x16& a0, const f32x16& a1) {
#pragma unroll
        for (int rg = 0; rg < 4; ++rg) {
            f32x4 v0 = {a0[4 * rg], a0[4 * rg + 1], a0[4 * rg + 2], a0[4 * rg + 3]};
            f32x4 v1 = {a1[4 * rg], a1[4 * rg + 1], a1[4 * rg + 2], a1[4 * rg + 3]};
            float* row = &dst[(slot * 64 + 32 * khalf + l32) * kRedRow + 8 * rg + 4 * hi];
            *(f32x4*)row = v0;
            *(f32x4*)(row + 32) = v1;
        }
    };
    // Projection variant (same page, the key launch's "dK = s (the sum) and dV
    // stored straight into a fused projection's gradient"): row p of the
    // token-major gradient takes K/V head kv's values at columns 64 kv + d of
    // the slice the pointers name, in binary32 and rounded to bfloat16.
    const size_t tok_row0 = (size_t)b * T + (size_t)kt * kTile;
    // With ch.accumulate (every query-row chunk after the first), the sums
    // are added to what the outputs hold: the earlier chunks' dK and dV.
    const bool acc = ch.accumulate != 0;
    auto store_proj = [&](const ProjectionOut& pr, int kk, int d4, f32x4 v) {
        const size_t at = (tok_row0 + kk) * (size_t)pr.width + kHeadDim * kv + d4;
        if (acc) v += *(const f32x4*)(pr.f32 + at);
        *(f32x4*)(pr.f32 + at) = v;
        *(uint2*)(pr.b16 + at) = pack_bf16x4(v[0], v[1], v[2], v[3]);
    };
    const bool proj = kproj.f32 != nullptr;
    to_lds(red, dkacc0, dkacc1);
    to_lds(red_v, dvacc0, dvacc1);
    __syncthreads();
    for (int idx = tid; idx < 64 * 16; idx += kThreads) {  // dK[key][d]: 16 float4s per key
        const int kk = idx >> 4, d4 = (idx & 15) * 4;
        f32x4 v = *(const f32x4*)&red[kk * kRedRow + d4];
#pragma unroll
        for (int g = 1; g < GW; ++g) v += *(const f32x4*)&red[(g * 64 + kk) * kRedRow + d4];
        v *= s;
        if (proj) {
            store_proj(kproj, kk, d4, v);
        } else {
            f32x4* out = (f32x4*)(dK + (key_row0 + kk) * kHeadDim + d4);
            if (acc) v += *out;
            *out = v;
        }
    }
    if (v_rows || proj) {
        for (int idx = tid; idx < 64 * 16; idx += kThreads) {  // dV[key][d]: 16 float4s per key
            const int kk = idx >> 4, d4 = (idx & 15) * 4;
            f32x4 v = *(const f32x4*)&red_v[kk * kRedRow + d4];
#pragma unroll
            for (int g = 1; g < GW; ++g) v += *(const f32x4*)&red_v[(g * 64 + kk) * kRedRow + d4];
            if (proj) {
                store_proj(vproj, kk, d4, v);
            } else {
                f32x4* out = (f32x4*)(dVt + (key_row0 + kk) * kHeadDim + d4);
                if (acc) v += *out;
                *out = v;
            }
        }
        return;
    }
    for (int idx = tid; idx < 64 * 16; idx += kThreads) {  // dV^T[d][key]: 16 float4s per d row
        const int d = idx >> 4, k4 = (idx & 15) * 4;
        f32x4 v;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            float a = red_v[(k4 + e) * kRedRow + d];
#pragma unroll
            for (int g = 1; g < GW; ++g) a += red_v[(g * 64 + k4 + e) * kRedRow + d];
            v[e] = a;
        }
        f32x4* out = (f32x4*)(dVt + (((size_t)b * KV + kv) * kHeadDim + d) * T + (size_t)kt * kTile + k4);
        if (acc) v += *out;
        *out = v;
    }
    };
    process(kt_first);
    if constexpr (!VARLEN) {
        if (kt_second >= 0) {
            __syncthreads();  // the first tile's group sums have been read from LDS
            process(kt_second);
        }
    }
}

// ---------------------------------------------------------------------------
// dQ pass.  One 256-thread workgroup per 128 queries of a query head (two dS
// tile rows); wave w owns 32 queries.  For each key tile up to the diagonal
// (the query pass's order) the K tile is staged in LDS for the four waves and
// each wave accumulates
//   dQ^T += K^T dS^T   (A = K^T by transposed LDS reads; B = dS^T: the key
//                       pass stores dS as its accumulators hold it, a lane's
//                       16 queries of one key, so each wave loads its 4 KB
//                       block of the tile as four coalesced 1 KB runs, writes
//                       it to its own LDS copy and reads it back transposed,
//                       8 keys of one query per lane)
// with the dS and K loads of the next four tiles in flight, since the pass
// streams the workspace from memory.  Each lane ends with 4-float runs of
// one query's dQ row: dQ = s * sum, which goes through LDS to be stored as
// whole rows.
// ---------------------------------------------------------------------------
constexpr int kDqWaves = 4;
constexpr int kDqRows = 32 * kDqWaves;
constexpr int kDqThreads = 64 * kDqWaves;
constexpr int kKTileHalves = kTile * kHeadDim;  // unpadded, chunk-swizzled
constexpr int kDsRunHalves = 512 + 32;          // a 1 KB dS run plus a 64-byte pad between its halves
constexpr int kDsBlockHalves = 4 * kDsRunHalves;

// dS tiles in flight per wave: the pass streams dS once from HBM, and the
// registers are the deepest buffer the chip has (five tiles are 80 VGPRs).
// K tiles travel with the same lead, straight into LDS (one buffer per tile
// in flight).  The hardware counts a wave's outstanding loads in issue order,
// so waiting for a K tile also waits for every dS load issued before it:
// only when both streams have the same lead does that wait cost nothing.
constexpr int kDqDepth = 5;
constexpr int kDqLead = kDqDepth - 1;             // tiles loaded ahead of use
constexpr int kDqVmPerStep = 2 + 4;               // per lane: K DMA, dS loads
// Loads issued after K tile kt + 1's DMA when step kt ends: that tile's four
// dS loads and the four steps since.  Waiting until no more than this many
// are outstanding means the tile has landed in LDS.
constexpr int kDqKWait = 4 + (kDqLead - 1) * kDqVmPerStep;
static_assert(kDqKWait == 22, "the s_waitcnt immediate below");

// ROT: the epilogue of the query pass's rotated variant (StreamingAttentionSM86
// page, "dQ = s (the sum), turned back by the inverse half-split rotation"):
// the scaled pair (x1, x2) of columns c and c + 32 at position p becomes
// (x1 cos + x2 sin, x2 cos - x1 sin) with the [T][32] tables' entry (p, c),
// each product rounded as the page's FMUL then FFMA, and is stored as
// bfloat16 at columns 64 h + c and 64 h + c + 32 of row p of the token-major
// [B][T][width] projection gradient; dQ itself is not written.
// PROJ: the projection variant's epilogue (same page, "dQ = s (the sum)
// stored straight into a fused projection's gradient"): the scaled dQ row
// goes to columns 64 h + c of row p of a token-major gradient, once in
// binary32 and once rounded to bfloat16, instead of the [B][H][T][64] plane.
enum { kDqPlain = 0, kDqRotated = 1, kDqProjection = 2 };
template <bool CAUSAL, bool VARLEN, int MODE>
__global__ __launch_bounds__(kDqThreads, 2) void sa_dq_kernel(const half_t* __restrict__ K,
                                                               const half_t* __restrict__ dS,
                                                               float* __restrict__ dQ,
                                                               const int32_t* __restrict__ seqlens, float s,
                                                               int T, int H, int KV, int n_qblk, int BH,
                                                               int block_order, Chunk ch, DqEpilogue rot) {
    __shared__ __attribute__((aligned(16))) half_t lds[kDqDepth][kKTileHalves];  // K tiles
    __shared__ __attribute__((aligned(16))) half_t dsl[kDqWaves][kDsBlockHalves];  // each wave's dS block

    const int tid = threadIdx.x, wave = wave_id(), lane = tid & 63;
    const int l32 = lane & 31, hi = lane >> 5;
    // Block -> (batch*head, query blocks).  Order 0: the pair (n - 1 - p, p),
    // whose causal walks add up to the same length, with the heads of one kv
    // head kept on one XCD.  Order 1: one query block per block, plain order.
    // The chunk's query blocks are blk_lo .. blk_lo + n_qblk - 1 (all of them
    // when the backward is not chunked).
    const int blk_lo = ch.q_lo / 2;
    int bh, n_items, items[2];
    if (VARLEN && block_order != kOrderPlain && BH / H <= kMaxRankedBatch) {
        // Variable lengths: the longest sequences' blocks first, then the
        // schedule's order within each sequence.
        const int per_b = H * (block_order == kOrderPairs ? (n_qblk + 1) / 2 : n_qblk);
        const int r = (int)blockIdx.x / per_b, rest = (int)blockIdx.x % per_b, k = rest / H;
        bh = batch_of_rank(seqlens, BH / H, T, r) * H + rest % H;
        items[0] = blk_lo + n_qblk - 1 - k;
        items[1] = blk_lo + k;
        n_items = (block_order == kOrderPairs && k < n_qblk - 1 - k) ? 2 : 1;
    } else if (block_order == kOrderPairs) {
        int pair;
        pair_schedule((int)blockIdx.x, (BH / H) * KV, H / KV, pair, bh);
        items[0] = blk_lo + n_qblk - 1 - pair;
        items[1] = blk_lo + pair;
        n_items = pair < n_qblk - 1 - pair ? 2 : 1;
    } else if (block_order == kOrderSingle) {  // one block of rows per block, the longest first
        items[0] = items[1] = blk_lo + n_qblk - 1 - (int)(blockIdx.x / BH);
        bh = (int)(blockIdx.x % BH);
        n_items = 1;
    } else {
        items[0] = items[1] = blk_lo + (int)(blockIdx.x % n_qblk);
        bh = (int)(blockIdx.x / n_qblk);
        n_items = 1;
    }
    const int b = bh / H, h = bh % H, kv = h / (H / KV);
    const int nt = T / kTile;
    const int len = VARLEN ? min(max(seqlens[b], 0), T) : T;
    const int ntl = VARLEN ? (len + kTile - 1) / kTile : nt;  // dS tile rows/cols in use
    const half_t* Kp = K + ((size_t)b * KV + kv) * (size_t)T * kHeadDim;

    // K DMA: wave w moves rows 8 (2 w + u) + lane / 8 (u = 0, 1) of a tile; a
    // lane's 16 bytes land at slot lane % 8 of its row, so it fetches the
    // row's chunk (lane % 8) ^ swz_key_k(row): LDS holds chunk c of a row at
    // c ^ swz_key_k(row).
    const int dma_row0 = 16 * wave + (lane >> 3), dma_row1 = dma_row0 + 8;
    const int dma_c0 = (lane & 7) ^ swz_key_k(dma_row0), dma_c1 = (lane & 7) ^ swz_key_k(dma_row1);
    auto dma_k = [&](int kt, int buf) {
        const half_t* src = Kp + (size_t)(kt * kTile) * kHeadDim;
        dma16(src + dma_row0 * kHeadDim + dma_c0 * 8, (char*)&lds[buf][(16 * wave) * kHeadDim]);
        dma16(src + dma_row1 * kHeadDim + dma_c1 * 8, (char*)&lds[buf][(16 * wave + 8) * kHeadDim]);
    };
    const int trr = (lane & 15) >> 2, trc = 16 * ((lane >> 4) & 1) + 4 * (lane & 3);
    // dS block in LDS: run u (quadrant kh = u / 2, query half u % 2) at
    // kDsRunHalves u; within a run, lane L's 16 bytes (key L % 32 of the
    // quadrant, queries of its half with (q / 4) % 2 = L / 32) at 8 L, plus
    // a 32-half pad for L >= 32.
    const int ds_slot = 8 * lane + ((lane >> 5) << 5);
    // Transposed read of k-step s4, keys +4 j (j = 0, 1): 16-lane group G
    // (= lane / 16) covers queries 16 (G % 2) + 0..15 and keys 8 (G / 2) +
    // 0..3 of the run's quadrant; its lane 4 row + cq names queries
    // 16 (G % 2) + 4 cq + 0..3 of key row `row`, stored in the run of query
    // half G % 2 at lane (cq % 2) 32 + key, word 4 (cq / 2).
    int ds_tr0[2];
    {
        const int G = lane >> 4, p = lane & 15, row = p >> 2, cq = p & 3;
        const int in_run = 8 * ((cq & 1) * 32 + 8 * (G >> 1) + row) + 32 * (cq & 1) + 4 * (cq >> 1);
#pragma unroll
        for (int kh = 0; kh < 2; ++kh) ds_tr0[kh] = kDsRunHalves * (2 * kh + (G & 1)) + in_run;
    }

    auto process = [&](const int qblk) {
        const int qt0 = 2 * qblk;
        const int qt_w = qt0 + (wave >> 1), qh = wave & 1;
        const int q = qblk * kDqRows + 32 * wave + l32;
        const bool wave_rows = qt_w < nt;

        int kt_end = CAUSAL ? min(qt0 + 2, nt) : nt;
        if (VARLEN) kt_end = min(kt_end, ntl);
        if (VARLEN && qt0 >= ntl) kt_end = 0;
        // Key tiles this wave reads: its dS row's tiles that exist.
        const int kt_end_w = wave_rows && qt_w < ntl ? (CAUSAL ? min(qt_w + 1, kt_end) : kt_end) : 0;
        const int kt_clamp = max(kt_end - 1, 0);

        // This wave's dS block of tile (qt_w, kt): the quadrants (qh, 0) and
        // (qh, 1), 4 KB at 2048 qh, loaded as four coalesced 1 KB runs (lane l
        // takes 16 bytes at 8 l of each).  Loads are issued on every path (see
        // below); only tiles up to kt_last of row qt_l are read, every other
        // load goes to the fixed block below (tiles past the item's last key
        // tile were never written).  With variable lengths, a wave whose rows
        // are all padding takes the block's first row as qt_l, so that the
        // address arithmetic stays in range, and reads only the fixed block.
        const int qt_l = (!VARLEN || kt_end_w > 0) ? min(qt_w, nt - 1) : qt0;
        const int kt_last = min(CAUSAL ? qt_l : nt - 1, max(kt_end - 1, 0));
        const half_t* dSw = dS + ((size_t)b * H + h) * (size_t)ch.tph * (kTile * kTile) +
                            (size_t)(2 * qh) * 1024 + 8 * lane +
                            ((CAUSAL ? (size_t)qt_l * (qt_l + 1) / 2 : (size_t)qt_l * nt) - (size_t)ch.tile0) *
                                (kTile * kTile);
        // Loads whose data goes unused (past the item's last key tile: the
        // lead's overrun at the end of a walk and the unrolled loop's padding
        // steps; every load of a wave whose rows are all padding) all read one
        // fixed block at the start of the workspace, which stays in every L2,
        // instead of streaming a tile again from memory.
        const half_t* dS_idle = dS + (size_t)(2 * qh) * 1024 + 8 * lane;
        const int kt_read = kt_end_w > 0 ? kt_last : -1;
        auto load_s = [&](int kt, half8 (&dst)[4]) {
            const half_t* t_ = kt <= kt_read ? dSw + (size_t)kt * (kTile * kTile) : dS_idle;
            dst[0] = gload16_stream_async(t_);
            dst[1] = gload16_stream_async(t_ + 512);
            dst[2] = gload16_stream_async(t_ + 1024);
            dst[3] = gload16_stream_async(t_ + 1536);
        };
        // Every step issues K's DMA then the dS loads, on every path, so a
        // wave's count of loads younger than any given one is fixed: the
        // waits below name it.  (The dS loads are invisible to the compiler,
        // whose own wait placement loses track of loop-carried loads.)
        auto issue = [&](int kt, half8 (&dst)[4]) {
            dma_k(min(kt, kt_clamp), kt % kDqDepth);
            asm volatile("" ::: "memory");
            load_s(kt, dst);
        };

        f32x16 acc0 = zero16(), acc1 = zero16();
        // An item whose rows are all padding (variable lengths) loads and walks
        // nothing: its rows are written as zeros below.  kt_end is the same
        // for every wave of the workgroup, so the barriers inside stay paired.
        if (!VARLEN || kt_end > 0) {
            // dS tile kt lives in register slot kt % 5 from step kt - 4 to step kt.
            half8 sl0[4], sl1[4], sl2[4], sl3[4], sl4[4];
            issue(0, sl0);
            issue(1, sl1);
            issue(2, sl2);
            issue(3, sl3);
            asm volatile("s_waitcnt vmcnt(22)" ::: "memory");  // K tile 0 (and older) landed
            __builtin_amdgcn_s_barrier();

            auto step = [&](const int kt, half8 (&cur)[4], half8 (&ahead)[4]) {
                issue(kt + kDqLead, ahead);
                // dS tile kt, issued four steps back: 24 loads are younger.  The
                // wait ties the slot and sits on every path, also where the tile
                // is not used (a padding step of the unrolled loop, or a tile past
                // this wave's rows): the compiler must not reuse or copy the
                // slot's registers (say, for the next step's addresses) while its
                // loads may still land in them.
                static_assert((kDqLead) * kDqVmPerStep == 24, "the s_waitcnt immediate below");
                asm volatile("s_waitcnt vmcnt(24)" : "+v"(cur[0]), "+v"(cur[1]), "+v"(cur[2]), "+v"(cur[3]));
                if (kt >= kt_end) return;  // padding step: loads only
                if (kt < kt_end_w) {
                    // The block goes through this wave's LDS copy (each 1 KB run
                    // padded by 64 bytes between its two 512-byte halves) and comes
                    // back transposed: lane (query l32, hi) gets the 8 keys of
                    // k-step s4, 16 s4 + 8 hi + 0..7, of its query.
                    half_t* dw = dsl[wave];
#pragma unroll
                    for (int u = 0; u < 4; ++u) lds_write16_async(dw + kDsRunHalves * u + ds_slot, cur[u]);
                    half4 g[8];
#pragma unroll
                    for (int s4 = 0; s4 < 4; ++s4) {
                        g[2 * s4] = lds_read_tr_async(dw + ds_tr0[s4 >> 1] + 128 * (s4 & 1));
                        g[2 * s4 + 1] = lds_read_tr_async(dw + ds_tr0[s4 >> 1] + 128 * (s4 & 1) + 32);
                    }
                    const half_t* Ks = lds[kt % kDqDepth];
                    half4 t[16];
#pragma unroll
                    for (int s4 = 0; s4 < 4; ++s4) {
                        // A = K^T: lane (d, hi) holds K[16 s4 + 8 hi + 0..7][d].
                        const int r0 = 16 * s4 + 8 * hi + trr;
                        t[4 * s4 + 0] = lds_read_tr_async(Ks + r0 * kHeadDim +
                                                          (((trc >> 3) ^ swz_key_k(r0)) << 3) + (trc & 7));
                        t[4 * s4 + 1] = lds_read_tr_async(Ks + (r0 + 4) * kHeadDim +
                                                          (((trc >> 3) ^ swz_key_k(r0 + 4)) << 3) + (trc & 7));
                        t[4 * s4 + 2] = lds_read_tr_async(Ks + r0 * kHeadDim +
                                                          ((((trc + 32) >> 3) ^ swz_key_k(r0)) << 3) + (trc & 7));
                        t[4 * s4 + 3] = lds_read_tr_async(Ks + (r0 + 4) * kHeadDim +
                                                          ((((trc + 32) >> 3) ^ swz_key_k(r0 + 4)) << 3) + (trc & 7));
                    }
                    lds_wait(t[0], t[1], t[2], t[3], t[4], t[5], t[6], t[7]);
                    lds_wait(t[8], t[9], t[10], t[11], t[12], t[13], t[14], t[15]);
                    lds_wait(g[0], g[1], g[2], g[3], g[4], g[5], g[6], g[7]);
                    if (VARLEN && (kt + 1) * kTile > len) {
                        // Keys at or past the length: the DMA brought whatever
                        // the padding holds; their dS is zero, so zero K too.
#pragma unroll
                        for (int s4 = 0; s4 < 4; ++s4)
#pragma unroll
                            for (int e = 0; e < 4; ++e) {
                                const int key = kt * kTile + 16 * s4 + 8 * hi + 4 * (e & 1) + 0;
#pragma unroll
                                for (int i = 0; i < 4; ++i)
                                    if (key + i >= len) t[4 * s4 + e][i] = (half_t)0.0f;
                            }
                    }
#pragma unroll
                    for (int s4 = 0; s4 < 4; ++s4) {
                        const half8 bs = cat(g[2 * s4], g[2 * s4 + 1]);
                        acc0 = mfma32(cat(t[4 * s4 + 0], t[4 * s4 + 1]), bs, acc0);
                        acc1 = mfma32(cat(t[4 * s4 + 2], t[4 * s4 + 3]), bs, acc1);
                    }
                }
                // K tile kt + 1 (and every older load) has landed in LDS; every
                // wave is done reading buffer kt % 5 before it is refilled.
                asm volatile("s_waitcnt vmcnt(22)" ::: "memory");
                __builtin_amdgcn_s_barrier();
            };
            static_assert(kDqDepth == 5, "five unrolled steps below");
            for (int kt = 0; kt < kt_end; kt += kDqDepth) {
                step(kt, sl0, sl4);
                step(kt + 1, sl1, sl0);
                step(kt + 2, sl2, sl1);
                step(kt + 3, sl3, sl2);
                step(kt + 4, sl4, sl3);
            }
            // The padding steps (and, with no tile to walk, the prologue) leave
            // dS loads in flight into slots nobody reads: the compiler, which does
            // not see them, would reuse those registers in the epilogue while a
            // late load could still land in them.  Drain them here, tying every
            // slot so that no register of theirs is reused before the wait.
            asm volatile("s_waitcnt vmcnt(0)"
                         : "+v"(sl0[0]), "+v"(sl0[1]), "+v"(sl0[2]), "+v"(sl0[3]), "+v"(sl1[0]), "+v"(sl1[1]),
                           "+v"(sl1[2]), "+v"(sl1[3]), "+v"(sl2[0]), "+v"(sl2[1]) :: "memory");
            asm volatile("s_waitcnt vmcnt(0)"
                         : "+v"(sl2[2]), "+v"(sl2[3]), "+v"(sl3[0]), "+v"(sl3[1]), "+v"(sl3[2]), "+v"(sl3[3]),
                           "+v"(sl4[0]), "+v"(sl4[1]), "+v"(sl4[2]), "+v"(sl4[3]) :: "memory");
        }
        if (!wave_rows) return;
        const float scale = (!VARLEN || q < len) ? s : 0.0f;
        if (MODE == kDqProjection) {
            const size_t row = ((size_t)b * T + q) * (size_t)rot.width + kHeadDim * h;
            float* o32 = rot.out32 + row;
            uint16_t* o16 = rot.out + row;
#pragma unroll
            for (int rg = 0; rg < 4; ++rg) {
                const int c0 = 8 * rg + 4 * hi;
                f32x4 v0 = {acc0[4 * rg], acc0[4 * rg + 1], acc0[4 * rg + 2], acc0[4 * rg + 3]};
                f32x4 v1 = {acc1[4 * rg], acc1[4 * rg + 1], acc1[4 * rg + 2], acc1[4 * rg + 3]};
                v0 *= scale;
                v1 *= scale;
                *(f32x4*)(o32 + c0) = v0;
                *(f32x4*)(o32 + 32 + c0) = v1;
                *(uint2*)(o16 + c0) = pack_bf16x4(v0[0], v0[1], v0[2], v0[3]);
                *(uint2*)(o16 + 32 + c0) = pack_bf16x4(v1[0], v1[1], v1[2], v1[3]);
            }
            return;
        }
        if (MODE == kDqRotated) {
            // Each lane holds columns c = 8 rg + 4 hi + 0..3 and c + 32 of its query's row.
            const float* cr = rot.cos + (size_t)q * 32;
            const float* sr = rot.sin + (size_t)q * 32;
            uint16_t* orow = rot.out + ((size_t)b * T + q) * (size_t)rot.width + kHeadDim * h;
#pragma unroll
            for (int rg = 0; rg < 4; ++rg) {
                const int c0 = 8 * rg + 4 * hi;
                const f32x4 cv = *(const f32x4*)(cr + c0), sv = *(const f32x4*)(sr + c0);
                float o1[4], o2[4];
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const float x1 = acc0[4 * rg + i] * scale, x2 = acc1[4 * rg + i] * scale;
                    o1[i] = __builtin_fmaf(x1, cv[i], x2 * sv[i]);
                    o2[i] = __builtin_fmaf(x2, cv[i], -(x1 * sv[i]));
                }
                *(uint2*)(orow + c0) = pack_bf16x4(o1[0], o1[1], o1[2], o1[3]);
                *(uint2*)(orow + 32 + c0) = pack_bf16x4(o2[0], o2[1], o2[2], o2[3]);
            }
            return;
        }
        // The wave's 32 dQ rows (8 KB, contiguous in the plane) go through
        // LDS so that each store writes four whole rows: row r sits in this
        // wave's own 16 rows of K buffer r / 8 (no other wave reads or fills
        // them, and the drain above has landed this wave's last K copies),
        // 256 bytes at (r % 8) 256, its 16-byte chunk c at c ^ (r % 16).
        // The stores are non-temporal: nothing here reads dQ again.
        char* stage = (char*)&lds[0][0] + 2048 * wave;
        auto chunk_at = [&](int r, int c) {
            return (f32x4*)(stage + (r >> 3) * (kKTileHalves * 2) + (r & 7) * 256 + ((c ^ (r & 15)) << 4));
        };
#pragma unroll
        for (int rg = 0; rg < 4; ++rg) {
            f32x4 v0 = {acc0[4 * rg], acc0[4 * rg + 1], acc0[4 * rg + 2], acc0[4 * rg + 3]};
            f32x4 v1 = {acc1[4 * rg], acc1[4 * rg + 1], acc1[4 * rg + 2], acc1[4 * rg + 3]};
            *chunk_at(l32, 2 * rg + hi) = v0 * scale;
            *chunk_at(l32, 8 + 2 * rg + hi) = v1 * scale;
        }
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
        __builtin_amdgcn_wave_barrier();
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
        float* dq = dQ + (((size_t)b * H + h) * T + (q - l32)) * kHeadDim;
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            const int r = 4 * j + (lane >> 4), c = lane & 15;
            __builtin_nontemporal_store(*chunk_at(r, c), (f32x4*)(dq + r * kHeadDim + 4 * c));
        }
    };
    process(items[0]);
    if (n_items == 2) {
        // Every DMA of the first item must land before the second refills
        // its buffers, and every wave must be past its last read.
        asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
        __builtin_amdgcn_s_barrier();
        process(items[1]);
    }
    // The padding steps leave DMAs into this workgroup's LDS and loads into
    // this wave's registers in flight: both must land before the wave ends.
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
}

template <bool CAUSAL, bool VARLEN>
void launch_key_gw(int GW, dim3 grid, hipStream_t stream, const half_t* Q, const half_t* K, const half_t* Vt,
                   const half_t* dO, const float* L, const float* D, half_t* dS, float* dK, float* dVt,
                   const int32_t* seqlens, float c, float s, int T, int H, int KV, int nkt, int BKV, int order,
                   const Chunk& ch, int v_rows, const ProjectionOut& kproj, const ProjectionOut& vproj) {
#define SA_KEY_LAUNCH(gw)                                                                                    \
    hipLaunchKernelGGL((sa_key_kernel<CAUSAL, VARLEN, gw>), grid, dim3(128 * gw), 0, stream, Q, K, Vt, dO, L, \
                       D, dS, dK, dVt, seqlens, c, s, T, H, KV, nkt, BKV, order, ch, v_rows, kproj, vproj)
    switch (GW) {
        case 4: SA_KEY_LAUNCH(4); break;
        case 3: SA_KEY_LAUNCH(3); break;
        case 2: SA_KEY_LAUNCH(2); break;
        default: SA_KEY_LAUNCH(1); break;
    }
#undef SA_KEY_LAUNCH
}

// Key-pass workgroups one CU holds at once: two waves per SIMD at 256
// registers (8 waves per CU) and the staging buffers' LDS (34 KB per wave pair).
int key_wgs_per_cu(int GW) { return GW >= 3 ? 1 : 4 / GW; }

// Wave pairs per key-pass workgroup: the largest divisor of the group size
// that is at most 4.
int key_gw(int G) {
    for (int gw = 4; gw > 1; --gw)
        if (G % gw == 0) return gw;
    return 1;
}

}  // namespace

size_t row_terms_blocks(const Shape& sh) {
    return (size_t)sh.batch * sh.heads * (size_t)(sh.T / kRowsPerBlock);
}
size_t key_pass_blocks(const Shape& sh) { return (size_t)sh.batch * sh.kv_heads * (sh.T / kTile); }
size_t dq_pass_blocks(const Shape& sh) {
    const size_t units = (size_t)sh.batch * sh.heads;
    const int n_qblk = (sh.T + kDqRows - 1) / kDqRows;
    return tile_schedule_blocks(tile_schedule(sh, units, n_qblk), units, n_qblk);
}

hipError_t launch_row_terms(const Shape& sh, const void* dO, const void* O, float* D, hipStream_t stream) {
    dim3 grid((unsigned)row_terms_blocks(sh)), block(kRowThreads);
    if (sh.seqlens)
        hipLaunchKernelGGL(sa_row_terms_kernel<true>, grid, block, 0, stream, (const half_t*)dO, (const half_t*)O,
                           D, sh.seqlens, sh.T, sh.heads);
    else
        hipLaunchKernelGGL(sa_row_terms_kernel<false>, grid, block, 0, stream, (const half_t*)dO,
                           (const half_t*)O, D, sh.seqlens, sh.T, sh.heads);
    return hipGetLastError();
}

// Key tiles a chunk's key pass launches: causal, only those below the
// chunk's last query tile (the later ones are finished by earlier chunks).
int chunk_key_tiles(const Shape& sh, const Chunk& ch) {
    const int nt = sh.T / kTile;
    return sh.causal ? min(ch.q_hi, nt) : nt;
}

hipError_t launch_key_pass_chunk(const Shape& sh, const Chunk& ch, const void* Q, const void* K, const void* Vt,
                                 const void* dO, const float* L, const float* D, void* dS, float c, float s,
                                 float* dK, float* dVt, const ProjectionOut& kproj, const ProjectionOut& vproj,
                                 hipStream_t stream) {
    const int nkt = chunk_key_tiles(sh, ch), BKV = sh.batch * sh.kv_heads;
    if (nkt <= 0) return hipSuccess;
    const int G = sh.heads / sh.kv_heads;
    // Grids too small for the chip (at most one workgroup per CU) with walks
    // long enough to share (T >= 512: at least 16 sub-tiles on key tile 0): a
    // group of one or two query heads walks its sub-tiles in 4 / G interleaved
    // phases, one wave pair each, four wave pairs per workgroup.
    const int GW = (G <= 2 && (size_t)BKV * nkt <= kChipCUs && sh.T >= 16 * kSubRows) ? 4 : key_gw(G);
    // Paired key tiles when single tiles take between one and two rounds of
    // the chip and the walks shrink linearly (causal, every chunk row down
    // to the diagonal): the pairs then fill it once, all of the same length.
    const size_t singles = (size_t)BKV * nkt, slots = (size_t)kChipCUs * key_wgs_per_cu(GW);
    const bool pairs = sh.causal && !sh.seqlens && sh.block_order == 0 && ch.q_lo == 0 && nkt >= 2 &&
                       singles > slots && singles <= 2 * slots;
    const int order = pairs ? kOrderKeyPairs : sh.block_order;
    dim3 grid((unsigned)(pairs ? (size_t)BKV * ((nkt + 1) / 2) : singles));
    auto go = [&](auto causal_tag, auto varlen_tag) {
        constexpr bool C = decltype(causal_tag)::value, V = decltype(varlen_tag)::value;
        launch_key_gw<C, V>(GW, grid, stream, (const half_t*)Q, (const half_t*)K, (const half_t*)Vt,
                            (const half_t*)dO, L, D, (half_t*)dS, dK, dVt, sh.seqlens, c, s, sh.T, sh.heads,
                            sh.kv_heads, nkt, BKV, order, ch, sh.v_rows, kproj, vproj);
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

hipError_t launch_key_pass_to(const Shape& sh, const void* Q, const void* K, const void* Vt, const void* dO,
                              const float* L, const float* D, void* dS, float c, float s, float* dK, float* dVt,
                              const ProjectionOut& kproj, const ProjectionOut& vproj, hipStream_t stream) {
    return launch_key_pass_chunk(sh, whole_problem(sh), Q, K, Vt, dO, L, D, dS, c, s, dK, dVt, kproj, vproj,
                                 stream);
}

hipError_t launch_key_pass(const Shape& sh, const void* Q, const void* K, const void* Vt, const void* dO,
                           const float* L, const float* D, void* dS, float c, float s, float* dK, float* dVt,
                           hipStream_t stream) {
    const ProjectionOut none{nullptr, nullptr, 0};
    return launch_key_pass_to(sh, Q, K, Vt, dO, L, D, dS, c, s, dK, dVt, none, none, stream);
}

hipError_t launch_key_pass_projection(const Shape& sh, const void* Q, const void* K, const void* Vt,
                                      const void* dO, const float* L, const float* D, void* dS, float c, float s,
                                      const ProjectionOut& kproj, const ProjectionOut& vproj, hipStream_t stream) {
    return launch_key_pass_to(sh, Q, K, Vt, dO, L, D, dS, c, s, nullptr, nullptr, kproj, vproj, stream);
}

template <int MODE>
hipError_t launch_dq_chunk(const Shape& sh, const Chunk& ch, const void* K, const void* dS, float s, float* dQ,
                           const DqEpilogue& rot, hipStream_t stream) {
    // The chunk's 128-row query blocks: q_lo is even, q_hi is even or the last tile.
    const int blk_lo = ch.q_lo / 2, blk_hi = (ch.q_hi + 1) / 2;
    const int n_qblk = blk_hi - blk_lo, BH = sh.batch * sh.heads;
    if (n_qblk <= 0) return hipSuccess;
    const int order = tile_schedule(sh, (size_t)BH, n_qblk);
    dim3 grid((unsigned)tile_schedule_blocks(order, (size_t)BH, n_qblk)), block(kDqThreads);
    auto go = [&](auto kern) {
        hipLaunchKernelGGL(kern, grid, block, 0, stream, (const half_t*)K, (const half_t*)dS, dQ, sh.seqlens, s,
                           sh.T, sh.heads, sh.kv_heads, n_qblk, BH, order, ch, rot);
    };
    if (sh.causal) {
        if (sh.seqlens) go(sa_dq_kernel<true, true, MODE>); else go(sa_dq_kernel<true, false, MODE>);
    } else {
        if (sh.seqlens) go(sa_dq_kernel<false, true, MODE>); else go(sa_dq_kernel<false, false, MODE>);
    }
    return hipGetLastError();
}

template <int MODE>
hipError_t launch_dq(const Shape& sh, const void* K, const void* dS, float s, float* dQ, const DqEpilogue& rot,
                     hipStream_t stream) {
    return launch_dq_chunk<MODE>(sh, whole_problem(sh), K, dS, s, dQ, rot, stream);
}

size_t min_chunk_bytes(const Shape& sh) { return largest_block_bytes(sh); }

hipError_t launch_key_dq_chunked(const Shape& sh, const void* Q, const void* K, const void* Vt, const void* dO,
                                 const float* L, const float* D, void* ws, size_t ws_bytes, float c, float s,
                                 float* dQ, float* dK, float* dVt, hipStream_t stream) {
    if (ws_bytes < min_chunk_bytes(sh)) return hipErrorInvalidValue;
    const ProjectionOut none{nullptr, nullptr, 0};
    const DqEpilogue plain{nullptr, nullptr, nullptr, nullptr, 0};
    // Chunks from the last rows down: each takes as many 128-row blocks as
    // fit in the workspace.  Causal, the first chunk reaches every key tile,
    // so every later one accumulates onto finished or started sums.
    int q_hi = sh.T / kTile;
    bool first = true;
    while (q_hi > 0) {
        const Chunk ch = next_chunk(sh, q_hi, ws_bytes, first);
        const int q_lo = ch.q_lo;
        hipError_t e = launch_key_pass_chunk(sh, ch, Q, K, Vt, dO, L, D, ws, c, s, dK, dVt, none, none, stream);
        if (e != hipSuccess) return e;
        if ((e = launch_dq_chunk<kDqPlain>(sh, ch, K, ws, s, dQ, plain, stream)) != hipSuccess) return e;
        first = false;
        q_hi = q_lo;
    }
    return hipSuccess;
}

hipError_t launch_dq_pass(const Shape& sh, const void* K, const void* dS, float s, float* dQ,
                          hipStream_t stream) {
    return launch_dq<kDqPlain>(sh, K, dS, s, dQ, DqEpilogue{nullptr, nullptr, nullptr, nullptr, 0}, stream);
}

hipError_t launch_dq_pass_rotated(const Shape& sh, const void* K, const void* dS, float s, const float* cos_t,
                                  const float* sin_t, void* dqkv, int width, hipStream_t stream) {
    return launch_dq<kDqRotated>(sh, K, dS, s, nullptr,
                                 DqEpilogue{cos_t, sin_t, (uint16_t*)dqkv, nullptr, width}, stream);
}

hipError_t launch_dq_pass_projection(const Shape& sh, const void* K, const void* dS, float s, const ProjectionOut& q,
                                     hipStream_t stream) {
    return launch_dq<kDqProjection>(sh, K, dS, s, nullptr,
                                    DqEpilogue{nullptr, nullptr, (uint16_t*)q.b16, q.f32, q.width}, stream);
}

}  // namespace sa
