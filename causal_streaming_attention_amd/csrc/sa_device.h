// sa_device.h -- gfx950 device helpers shared by the attention kernels.
//
// Wave64 MFMA v_mfma_f32_32x32x16_f16 operand geometry (lane l, l32 = l % 32,
// hi = l / 32):
//   A (32 x 16):  lane holds A[l32][8 hi + t],        t = 0..7
//   B (16 x 32):  lane holds B[8 hi + t][l32],        t = 0..7
//   C (32 x 32):  lane holds C[8 (r/4) + 4 hi + r%4][l32], r = 0..15
// ds_read_b64_tr_b16 (per 16-lane group): the lane with index
// 4 * row + chunk (within the group) names 4 consecutive halves at
// (row, 4 * chunk) of the group's 4 x 16 block; afterwards lane i of the
// group holds that block's column i, rows 0..3.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace sa {

typedef _Float16 half_t;
typedef _Float16 half4 __attribute__((ext_vector_type(4)));
typedef _Float16 half8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef __fp16 fp16x4_raw __attribute__((__vector_size__(4 * sizeof(__fp16))));

constexpr int kHeadDim = 64;
constexpr int kTile = 64;          // keys per tile and rows per dS tile
constexpr int kLdsRow = 72;        // padded LDS row, in halves (144 bytes)
constexpr float kNegInf = -__builtin_huge_valf();

__device__ __forceinline__ f32x16 mfma32(const half8& a, const half8& b, const f32x16& c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ f32x16 zero16() {
    f32x16 z;
#pragma unroll
    for (int i = 0; i < 16; ++i) z[i] = 0.0f;
    return z;
}

// 2^x on the transcendental unit (v_exp_f32): 2^-inf = 0.
__device__ __forceinline__ float exp2_fast(float x) { return __builtin_amdgcn_exp2f(x); }
// log2 x (v_log_f32) and 1/x (v_rcp_f32), about 1 ulp.
__device__ __forceinline__ float log2_fast(float x) { return __builtin_amdgcn_logf(x); }
__device__ __forceinline__ float rcp_fast(float x) { return __builtin_amdgcn_rcpf(x); }

// Reductions across the two wave halves (lane l with lane l ^ 32) by one
// v_permlane32_swap: between them its two results hold both halves' values in
// every lane, so max and sum are exact and identical in all 64 lanes.
__device__ __forceinline__ float max_halves(float x) {
    auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float sum_halves(float x) {
    auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// s_waitcnt vmcnt(0) as a compiler-visible wait (expcnt and lgkmcnt left at
// their maxima): the wait-insertion pass folds it into its own count, so
// loads that are known to have landed stop being treated as outstanding.
__device__ __forceinline__ void vm_wait_all() { __builtin_amdgcn_s_waitcnt(0x0F70); }

// Block schedule shared by the kernels whose per-tile work follows the causal
// triangle.  Tile t and tile n - 1 - t form a pair whose two walks add up to
// the same length for every t, so a grid of (pairs x units) blocks, each doing
// its pair's two tiles, is balanced with no tail of short blocks.  A unit is a
// (batch, head) or a (batch, kv head); units come in groups that read the same
// K/V (the query heads of one kv head).  The chip hands workgroups to its 8
// XCDs round-robin by index, each XCD with its own L2: when the group count is
// a multiple of 8, XCD x is given whole groups (x, x + 8, ...), so a group's
// K/V is cached in one L2 instead of in all eight.
constexpr int kXcds = 8;
__device__ __forceinline__ void pair_schedule(int block, int n_groups, int group_size, int& pair, int& unit) {
    const int n_units = n_groups * group_size;
    if (n_groups % kXcds == 0) {
        const int xcd = block % kXcds, k = block / kXcds;
        const int units_per_xcd = (n_groups / kXcds) * group_size;
        pair = k / units_per_xcd;
        const int r = k % units_per_xcd;
        unit = ((r / group_size) * kXcds + xcd) * group_size + r % group_size;
    } else {
        pair = block / n_units;
        unit = block % n_units;
    }
}

// Variable-length batches of at most 64 sequences: the batch entry of rank r
// when the entries are ordered by descending sequence length (ties by index),
// so that block indices can hand out the longest sequences' work first.
// Every lane of the wave returns the same value.
constexpr int kMaxRankedBatch = 64;
__device__ __forceinline__ int batch_of_rank(const int32_t* seqlens, int B, int T, int r) {
    const int lane = threadIdx.x & 63;
    const int mine = lane < B ? min(max(seqlens[lane], 0), T) : -1;
    int rank = 0;
    for (int j = 0; j < B; ++j) {
        const int other = __builtin_amdgcn_readlane(mine, j);
        rank += (other > mine || (other == mine && j < lane)) ? 1 : 0;
    }
    const unsigned long long hit = __builtin_amdgcn_ballot_w64(lane < B && rank == r);
    return (int)__builtin_ctzll(hit);
}

// Word 3 of a raw buffer resource on gfx950 (32-bit data format, no swizzle,
// no index stride): loads address base + voffset + soffset, bounded by the
// record count in bytes.
constexpr int kBufferRsrcWord3 = 0x00020000;

// Round to nearest even bfloat16: the upper half of the binary32 word after
// adding half an ulp of the kept part, ties going to the even one (inputs are
// finite).
__device__ __forceinline__ uint32_t bf16_bits(float x) {
    const uint32_t u = __float_as_uint(x);
    return (u + 0x7FFFu + ((u >> 16) & 1u)) >> 16;
}
__device__ __forceinline__ uint2 pack_bf16x4(float a, float b, float c, float d) {
    return make_uint2(bf16_bits(a) | (bf16_bits(b) << 16), bf16_bits(c) | (bf16_bits(d) << 16));
}

// Round to nearest even binary16.
__device__ __forceinline__ half_t to_half(float x) { return (half_t)x; }

typedef _Float16 half2_t __attribute__((ext_vector_type(2)));
// Two floats rounded to nearest even binary16 and packed (v_cvt_pk_f16_f32),
// the first in the low half.
__device__ __forceinline__ uint32_t pack_half2(float lo, float hi) {
    half2_t h;
    h[0] = (half_t)lo;
    h[1] = (half_t)hi;
    return __builtin_bit_cast(uint32_t, h);
}
__device__ __forceinline__ half8 half8_from_words(uint32_t w0, uint32_t w1, uint32_t w2, uint32_t w3) {
    uint4 u = make_uint4(w0, w1, w2, w3);
    return __builtin_bit_cast(half8, u);
}

// The wave index within the workgroup, as a scalar (wave-uniform) value.
__device__ __forceinline__ int wave_id() { return __builtin_amdgcn_readfirstlane(threadIdx.x >> 6); }

typedef __attribute__((address_space(3))) fp16x4_raw lds_fp16x4;

// ds_read_b64_tr_b16 at an LDS element pointer (must point into __shared__ memory).
__device__ __forceinline__ half4 lds_read_tr(const half_t* p) {
    fp16x4_raw v = __builtin_amdgcn_ds_read_tr16_b64_v4f16(
        (lds_fp16x4*)((__attribute__((address_space(3))) half_t*)(p)));
    return __builtin_bit_cast(half4, v);
}

// The same transposed read issued as inline assembly: the compiler does not
// track it, so it adds no wait for unrelated in-flight global-to-LDS loads.
// The caller must wait with lds_wait() (tying the results) before using them.
__device__ __forceinline__ half4 lds_read_tr_async(const half_t* p) {
    half4 r;
    const uint32_t addr = (uint32_t)(uintptr_t)(__attribute__((address_space(3))) const half_t*)(p);
    asm volatile("ds_read_b64_tr_b16 %0, %1" : "=v"(r) : "v"(addr) : "memory");
    return r;
}
// The same read at LDS byte address addr + OFF, the constant part of the
// address in the instruction's offset field.
template <int OFF>
__device__ __forceinline__ half4 lds_read_tr_at(uint32_t addr) {
    static_assert(OFF >= 0 && OFF < 65536, "DS offset field is 16 bits");
    half4 r;
    asm volatile("ds_read_b64_tr_b16 %0, %1 offset:%2" : "=v"(r) : "v"(addr), "i"(OFF) : "memory");
    return r;
}
// LDS byte address of an element pointer into __shared__ memory.
__device__ __forceinline__ uint32_t lds_addr(const void* p) {
    return (uint32_t)(uintptr_t)(__attribute__((address_space(3))) const char*)(p);
}
// An 8-byte LDS write the compiler does not see as one (no waits are placed
// for it); a later asm LDS read and its lgkmcnt wait order after it.
__device__ __forceinline__ void lds_write8_async(half_t* p, uint2 v) {
    const uint32_t addr = (uint32_t)(uintptr_t)(__attribute__((address_space(3))) half_t*)(p);
    asm volatile("ds_write_b64 %0, %1" : : "v"(addr), "v"(v) : "memory");
}
// A 16-byte LDS write the compiler does not see as one (as lds_write8_async).
__device__ __forceinline__ void lds_write16_async(half_t* p, half8 v) {
    const uint32_t addr = (uint32_t)(uintptr_t)(__attribute__((address_space(3))) half_t*)(p);
    asm volatile("ds_write_b128 %0, %1" : : "v"(addr), "v"(v) : "memory");
}
// A 16-byte non-temporal global load (data streamed once) that the compiler
// does not track: the caller must wait for it with an s_waitcnt vmcnt that
// ties the result (asm "+v"), counting every vector memory instruction
// issued after it.
__device__ __forceinline__ half8 gload16_stream_async(const void* p) {
    half8 r;
    asm volatile("global_load_dwordx4 %0, %1, off nt" : "=v"(r) : "v"(p) : "memory");
    return r;
}
// Wait for every outstanding LDS read of this wave; the operands are tied so
// no use of them can be scheduled before the wait.
__device__ __forceinline__ void lds_wait(half4& a, half4& b, half4& c, half4& d, half4& e, half4& f, half4& g,
                                         half4& h) {
    asm volatile("s_waitcnt lgkmcnt(0)" : "+v"(a), "+v"(b), "+v"(c), "+v"(d), "+v"(e), "+v"(f), "+v"(g), "+v"(h));
}

__device__ __forceinline__ void lds_wait4(half4& a, half4& b, half4& c, half4& d) {
    asm volatile("s_waitcnt lgkmcnt(0)" : "+v"(a), "+v"(b), "+v"(c), "+v"(d));
}

__device__ __forceinline__ half8 cat(const half4& lo, const half4& hi) {
    half8 r;
    r[0] = lo[0]; r[1] = lo[1]; r[2] = lo[2]; r[3] = lo[3];
    r[4] = hi[0]; r[5] = hi[1]; r[6] = hi[2]; r[7] = hi[3];
    return r;
}

// Per-lane element offset, inside a row-major LDS block with row stride
// kLdsRow, that a transposed read names so that lane l of a wave receives
// column (col0 + 16 * ((l / 16) % 2) + l % 16) at rows row0(l) + 0..3, where
// row0 = rowA for lanes 0..31 and rowB for lanes 32..63.
__device__ __forceinline__ int tr_offset(int lane, int rowA, int rowB, int col0, int stride = kLdsRow) {
    int row0 = (lane & 32) ? rowB : rowA;
    int r = (lane & 15) >> 2, chunk = lane & 3;
    return (row0 + r) * stride + col0 + 16 * ((lane >> 4) & 1) + 4 * chunk;
}

}  // namespace sa
