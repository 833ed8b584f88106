// fa_common.h -- gfx950 building blocks shared by the attention kernels.
//
// MFMA lane layouts used throughout (v_mfma_f32_32x32x16_bf16, D = A B + C,
// A is 32x16, B is 16x32, D is 32x32; lane l in 0..63, h = l / 32):
//   A operand: lane l holds A[l % 32][8h .. 8h + 7]        (8 bf16, 16 bytes)
//   B operand: lane l holds B[8h .. 8h + 7][l % 32]
//   D:         lane l, register r (0..15) holds D[8(r/4) + 4h + r%4][l % 32]
// so an accumulator keeps its column index on the lanes and its row index
// in the registers.  An accumulator D[m][n] can feed the next MFMA directly
// as the B operand B[k = m][n] (or A operand A[m' = n][k = m]) once its
// 16-register block is split into two k-steps: k-step t uses registers
// 8t .. 8t+7, i.e. MFMA k index 8h + j stands for row 16t + 8(j/4) + 4h +
// j%4 of the accumulator.  The other operand of that MFMA must follow the
// same row order ("k permutation").
//
// ds_read_b64_tr_b16 (gfx950 transposing LDS read): within each group of 16
// lanes, lane L reads 4 consecutive 16-bit values w_L[0..3]; lane i of the
// group then receives (w_{i/4 + 0}[i%4], w_{i/4 + 4}[i%4], w_{i/4 + 8}[i%4],
// w_{i/4 + 12}[i%4]).  Pointing lane L at row k0 + L/4, columns n0 + 4(L%4)
// of a row-major tile hands lane i column n0 + i, rows k0 .. k0+3: the
// column access an MFMA operand needs, from a row-major tile.
//
// LDS tiles are row-major with 16-byte chunks XOR-swizzled per row so that
// both access kinds are free of bank conflicts (64 banks x 4 bytes):
//   * 16-byte row reads of 16 consecutive rows at one logical chunk, and
//   * transposing reads of 4 consecutive rows x 64 bytes per half wave.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

typedef __bf16 fa_bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 fa_bf16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 fa_bf16x2 __attribute__((ext_vector_type(2)));
typedef float fa_f32x16 __attribute__((ext_vector_type(16)));
typedef float fa_f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t fa_u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t fa_u32x2 __attribute__((ext_vector_type(2)));
typedef __attribute__((address_space(3))) char fa_lds_char;
typedef __amdgpu_buffer_rsrc_t fa_rsrc;

#define FA_LOG2E 1.4426950408889634f
#define FA_LN2 0.6931471805599453f

namespace fa {

__device__ __forceinline__ fa_f32x16 mfma32(fa_u32x4 a, fa_u32x4 b, fa_f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(fa_bf16x8, a),
                                                   __builtin_bit_cast(fa_bf16x8, b), c, 0, 0, 0);
}

__device__ __forceinline__ fa_f32x16 zero16() {
    fa_f32x16 z;
#pragma unroll
    for (int i = 0; i < 16; ++i) z[i] = 0.0f;
    return z;
}

// Two fp32 -> packed bf16 (round to nearest even), low half = a.
__device__ __forceinline__ uint32_t pack_bf16(float a, float b) {
    fa_bf16x2 v = {(__bf16)a, (__bf16)b};
    return __builtin_bit_cast(uint32_t, v);
}

// Raw buffer resources.  A buffer access whose byte offset lies at or past
// num_records is dropped by the hardware (loads return 0, stores and atomics
// do nothing), which replaces per-row bounds branches for ragged tails.
__device__ __forceinline__ fa_rsrc make_rsrc(const void *base, uint32_t num_bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), 0, (int)num_bytes, 0x00020000);
}

__device__ __forceinline__ fa_u32x4 buf_load16(fa_rsrc r, uint32_t off) {
    return __builtin_bit_cast(fa_u32x4, __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 0));
}

__device__ __forceinline__ float buf_load4f(fa_rsrc r, uint32_t off) {
    return __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(r, off, 0, 0));
}

__device__ __forceinline__ void buf_store16(fa_rsrc r, uint32_t off, fa_u32x4 v) {
    __builtin_amdgcn_raw_buffer_store_b128(v, r, off, 0, 0);
}

__device__ __forceinline__ void buf_store8(fa_rsrc r, uint32_t off, fa_u32x2 v) {
    __builtin_amdgcn_raw_buffer_store_b64(__builtin_bit_cast(fa_u32x2, v), r, off, 0, 0);
}

__device__ __forceinline__ void buf_store4(fa_rsrc r, uint32_t off, uint32_t v) {
    __builtin_amdgcn_raw_buffer_store_b32(v, r, off, 0, 0);
}

__device__ __forceinline__ void buf_store2(fa_rsrc r, uint32_t off, uint16_t v) {
    __builtin_amdgcn_raw_buffer_store_b16(v, r, off, 0, 0);
}

__device__ __forceinline__ void buf_atomic_add(fa_rsrc r, uint32_t off, float v) {
    __builtin_amdgcn_raw_ptr_buffer_atomic_fadd_f32(v, r, off, 0, 0);
}

// LDS poison (debug build, -DFA_LDS_POISON): every direct copy first fills
// its destination with all-ones bytes (NaN as fp32 and as bf16), waits for
// that write, then copies.  A wave that reads a stage while another wave
// refills it, or before its copy has landed, reads NaN instead of plausible
// stale data, so a barrier out of place shows up as a changed result.
// Nothing else differs: the arithmetic, and so every output bit, is that of
// the normal build.
__device__ __forceinline__ void lds_poison(fa_lds_char *lds_wave_base, int bytes) {
#ifdef FA_LDS_POISON
    fa_lds_char *p = lds_wave_base + (threadIdx.x & 63) * bytes;
    if (bytes == 16) {
        const fa_u32x4 ones = {~0u, ~0u, ~0u, ~0u};
        *(__attribute__((address_space(3))) fa_u32x4 *)p = ones;
    } else {
        *(__attribute__((address_space(3))) uint32_t *)p = ~0u;
    }
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
#else
    (void)lds_wave_base;
    (void)bytes;
#endif
}

// Direct global -> LDS copy (buffer_load ... lds): every lane of the wave
// fetches BYTES (4 or 16) at its own byte offset and the hardware stores them
// at lds_wave_base + lane * BYTES.  lds_wave_base must be wave-uniform.
template <int BYTES>
__device__ __forceinline__ void buf_load_lds(fa_rsrc r, fa_lds_char *lds_wave_base, uint32_t off) {
    lds_poison(lds_wave_base, BYTES);
    auto *dst = (__attribute__((address_space(3))) void *)lds_wave_base;
    if constexpr (BYTES == 16) {
        __builtin_amdgcn_raw_ptr_buffer_load_lds(r, dst, 16, off, 0, 0, 0);
    } else {
        static_assert(BYTES == 4, "4- or 16-byte lanes");
        __builtin_amdgcn_raw_ptr_buffer_load_lds(r, dst, 4, off, 0, 0, 0);
    }
}

// Index of the calling wave in its workgroup, as a wave-uniform (scalar) value.
__device__ __forceinline__ int wave_id() { return __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6)); }

// Wait until every outstanding vector-memory operation of this wave is done.
__device__ __forceinline__ void wait_vmem() { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); }

__device__ __forceinline__ float bf16_lo(uint32_t u) { return __uint_as_float(u << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t u) { return __uint_as_float(u & 0xFFFF0000u); }

// Swizzle of the 16-byte chunk index within a row of a row-major LDS tile.
// NCH = chunks per row: 16 (256-byte rows) or 8 (128-byte rows).
template <int NCH>
__device__ __forceinline__ int swz(int row) {
    if constexpr (NCH == 16) {
        return ((row & 3) << 2) | ((row >> 2) & 3);
    } else {
        static_assert(NCH == 8, "rows of 128 or 256 bytes");
        return (((row >> 1) & 1) << 2) | ((row >> 2) & 3);
    }
}

// Copy ROWS rows of a row-major global matrix (rows of NCH*16 bytes, PITCH
// bytes apart, starting at byte offset row0 * PITCH of the resource) into a
// swizzled LDS tile with NW waves (w = wave index, wave-uniform), straight
// from memory to LDS.  Each wave instruction fills 1 KB of LDS contiguously,
// so the swizzle is applied on the global side: the lane that owns physical
// chunk pc of a row fetches logical chunk pc ^ swz(row).  Rows past the
// resource end arrive as zeros.
template <int NCH, int ROWS, int NW = 4>
__device__ __forceinline__ void tile_to_lds_pitched(fa_rsrc r, int row0, uint32_t pitch,
                                                    fa_lds_char *tile, int w, int lane) {
    constexpr int ROWB = NCH * 16;
    constexpr int ROWS_PER_INST = 1024 / ROWB;
    constexpr int INSTS = ROWS * ROWB / 1024;   // wave instructions for the tile
    static_assert(INSTS % NW == 0, "tile must split evenly over the waves");
#pragma unroll
    for (int k = 0; k < INSTS / NW; ++k) {
        const int inst = w + NW * k;
        const int row = inst * ROWS_PER_INST + lane / NCH;
        const int pc = lane % NCH;
        const int c = pc ^ swz<NCH>(row);
        const uint32_t goff = (uint32_t)(row0 + row) * pitch + c * 16;
        buf_load_lds<16>(r, tile + inst * 1024, goff);
    }
}

// The same for densely packed rows (pitch = row length).
template <int NCH, int ROWS, int NW = 4>
__device__ __forceinline__ void tile_to_lds(fa_rsrc r, int row0, fa_lds_char *tile, int w, int lane) {
    tile_to_lds_pitched<NCH, ROWS, NW>(r, row0, NCH * 16, tile, w, lane);
}

// Byte offset of (row, byte-in-row) inside a swizzled tile with NCH chunks per row.
template <int NCH>
__device__ __forceinline__ int tile_off(int row, int byte) {
    return row * (NCH * 16) + ((((byte >> 4) ^ swz<NCH>(row))) << 4) + (byte & 15);
}

__device__ __forceinline__ fa_u32x4 lds_read16(const fa_lds_char *base, int off) {
    return *(const __attribute__((address_space(3))) fa_u32x4 *)(base + off);
}

__device__ __forceinline__ void lds_write16(fa_lds_char *base, int off, fa_u32x4 v) {
    *(__attribute__((address_space(3))) fa_u32x4 *)(base + off) = v;
}

__device__ __forceinline__ void lds_write8(fa_lds_char *base, int off, fa_u32x2 v) {
    *(__attribute__((address_space(3))) fa_u32x2 *)(base + off) = v;
}

__device__ __forceinline__ fa_u32x2 lds_read_tr(const fa_lds_char *base, int off) {
    fa_bf16x4 v = __builtin_amdgcn_ds_read_tr16_b64_v4bf16(
        (__attribute__((address_space(3))) fa_bf16x4 *)(base + off));
    return __builtin_bit_cast(fa_u32x2, v);
}

// MFMA operand (8 bf16 of one column, rows k0 .. k0+7 in the given order)
// from a row-major swizzled tile via two transposing reads.  The lane's
// column is col_base + (lane % 32); rows are row_a + 0..3 (first half) and
// row_b + 0..3 (second half), both multiples of 4.
template <int NCH>
__device__ __forceinline__ fa_u32x4 operand_tr(const fa_lds_char *tile, int row_a, int row_b,
                                               int col_base, int lane) {
    const int L = lane & 15;
    const int col = col_base + ((lane >> 4) & 1) * 16 + (L & 3) * 4;  // first of 4 columns
    const fa_u32x2 lo = lds_read_tr(tile, tile_off<NCH>(row_a + (L >> 2), col * 2));
    const fa_u32x2 hi = lds_read_tr(tile, tile_off<NCH>(row_b + (L >> 2), col * 2));
    fa_u32x4 r = {lo[0], lo[1], hi[0], hi[1]};
    return r;
}

// v_permlane32_swap on (x, x) returns, in each lane l, the pair
// {x[l], x[l ^ 32]} (which of the two outputs holds which depends on the
// half); a commutative combine of the pair is the same in both halves.
__device__ __forceinline__ float max_halves(float x) {
    auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}

__device__ __forceinline__ float sum_halves(float x) {
    auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

}  // namespace fa
