// lds_tiles.hpp -- helpers shared by the kernels that stage token rows in LDS and
// read them back as MFMA operands (fused.hip, pair.hip).
#pragma once

#include "common.hpp"

namespace mhla {

// Physical 16-byte unit of chunk `chunk` of row `row` in an LDS array of `cpr` 16-byte
// chunks per row, XOR-swizzled so that eight consecutive rows read at one chunk fall
// on eight different groups of four banks: inside the row when rows are whole 128-byte
// lines (cpr a multiple of 8), else inside each aligned 128-byte line of the array.
__device__ __forceinline__ int swz(int row, int chunk, int cpr) {
    if ((cpr & 7) == 0) return row * cpr + (chunk ^ (row & 7));
    const int u = row * cpr + chunk, line = u >> 3;
    return (line << 3) | ((u & 7) ^ (line & 7));
}

// The (row, chunk) that swz maps to 16-byte unit L: its inverse.
__device__ __forceinline__ void unswz(int L, int cpr, int& row, int& chunk) {
    if ((cpr & 7) == 0) {
        row = L / cpr;
        chunk = (L % cpr) ^ (row & 7);
    } else {
        const int line = L >> 3, u = (line << 3) | ((L & 7) ^ (line & 7));
        row = u / cpr;
        chunk = u % cpr;
    }
}

__device__ __forceinline__ float lo_bf16(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float hi_bf16(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

// x of lane n ^ 8 of the same 16-lane group (DPP row rotate by 8: a VALU move, no LDS).
__device__ __forceinline__ float swap_half_row(float x) {
    return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(x), 0x128, 0xF, 0xF, false));
}

// Two 16 x 16 float32 output tiles c and c + 1 that share the 128-byte lines of their 16
// rows (lane (g, n) holds columns 4g .. 4g + 3 of row n of each) regrouped so that each
// of two 16-byte stores per lane writes whole lines: `top` holds rows 0 .. 7 (lanes n < 8
// tile c of row n, lanes n >= 8 tile c + 1 of row n - 8), `bottom` rows 8 .. 15 (lanes
// n < 8 tile c of row n + 8, lanes n >= 8 tile c + 1 of row n).  Lane (g, n) stores
// both at column 16 (c + n / 8) + 4g, rows n % 8 and 8 + n % 8.
__device__ __forceinline__ void whole_lines(const f32x4& y0, const f32x4& y1, int n, f32x4& top, f32x4& bottom) {
    const bool lo = n < 8;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
        const float u = swap_half_row(y1[e]), v = swap_half_row(y0[e]);
        top[e] = lo ? y0[e] : u;
        bottom[e] = lo ? v : y1[e];
    }
}

// phi of the two bf16 values of a word, packed back to bf16.
__device__ __forceinline__ uint32_t phi_pair(uint32_t w) {
    return pack_bf16(phi_fast(lo_bf16(w)), phi_fast(hi_bf16(w)));
}

// 8 bytes at LDS byte address `a`, transposed across each 16-lane group: lane i gets,
// as element e, element i % 4 of what lane 4e + i / 4 of its group addressed (gfx950
// ds_read_b64_tr_b16).
__device__ __forceinline__ s16x4 lds_read_tr16(const unsigned char* a) {
    return __builtin_amdgcn_ds_read_tr16_b64_v4i16(
        (__attribute__((address_space(3))) s16x4*)(const_cast<unsigned char*>(a)));
}

// A 16 x 32 MFMA operand (16x16x32: lane (g, n) holds row n, k-slots 8g .. 8g + 7) read
// transposed from a row-major swizzled bf16 array of `cpr` 16-byte pieces per row:
// operand row n is array column c0 + n, k-slot 8g + 4hh + e is array row r0 + 16hh + 4g
// + e.  Each 16-lane group addresses rows r0 + 16hh + 4g + n / 4, columns c0 + 4 (n % 4)
// .. +3 (the transposing read hands lane n element n % 4 of 4 such rows).
__device__ __forceinline__ bf16x8 lds_operand_t(const unsigned char* arr, int r0, int c0, int cpr, int g, int n) {
    s16x4 half[2];
#pragma unroll
    for (int hh = 0; hh < 2; ++hh) {
        const int row = r0 + 16 * hh + 4 * g + (n >> 2), col = c0 + 4 * (n & 3);
        half[hh] = lds_read_tr16(arr + 16 * swz(row, col >> 3, cpr) + 2 * (col & 7));
    }
    return __builtin_bit_cast(bf16x8, __builtin_shufflevector(half[0], half[1], 0, 1, 2, 3, 4, 5, 6, 7));
}

}  // namespace mhla
