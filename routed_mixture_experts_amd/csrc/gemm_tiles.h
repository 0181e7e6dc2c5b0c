// Helpers shared by the GEMM kernels: the tile list walk (XCD-aware and
// banded), the gathered row map, and explicit s_waitcnt forms.
#pragma once

#include "common.h"

namespace moe {
namespace tiles {

typedef __attribute__((address_space(3))) void* lds_ptr_t;

__device__ __forceinline__ int xcd_remap(int i, int total) {
    const int xcd = i & 7, local = i >> 3;
    const int per = total >> 3, rem = total & 7;
    return xcd * per + min(xcd, rem) + local;
}

struct TileCoord {
    int group, row0, row1, nt;
};

// Row tiles per band in the launch order of one group's tiles.
constexpr int kBandRows = 4;

// Position o of a block of cnt row tiles x ntn column tiles, taken in bands of
// kBandRows row tiles; inside a band the row tile varies fastest, so the
// workgroups resident on one XCD at a time form a kBandRows x (32 /
// kBandRows) block and reuse both operands' K slices from its L2.
__device__ __forceinline__ void band_order(int o, int cnt, int ntn, int& mt, int& nt) {
    const int band = o / (kBandRows * ntn);
    const int in_band = o - band * kBandRows * ntn;
    const int rows = min(kBandRows, cnt - band * kBandRows);
    nt = in_band / rows;
    mt = band * kBandRows + (in_band - nt * rows);
}

// Returns false when this workgroup has no tile (grids are sized from an
// upper bound of the tile count).
__device__ __forceinline__ bool fetch_tile(const GemmArgs& g, int tile_m, int ntn, TileCoord& c) {
    const int nm = g.tiles ? *g.num_tiles : (g.M + tile_m - 1) / tile_m;
    const int total = nm * ntn;
    const int i = blockIdx.x;
    if (i >= total) return false;
    const int lid = xcd_remap(i, total);
    int mt;
    if (g.tiles) {
        // the tiles of one group are contiguous: tile lid / ntn belongs to the
        // group whose block of count * ntn workgroups holds lid
        const Tile t0 = g.tiles[lid / ntn];
        const int first = __builtin_amdgcn_readfirstlane(t0.first);
        const int cnt = __builtin_amdgcn_readfirstlane(t0.count);
        band_order(lid - first * ntn, cnt, ntn, mt, c.nt);
        const Tile t = g.tiles[first + mt];
        // the tile is the same for the whole workgroup: keep it in SGPRs so
        // that every branch on it is a scalar branch
        c.group = __builtin_amdgcn_readfirstlane(t.group);
        c.row0 = __builtin_amdgcn_readfirstlane(t.row0);
        c.row1 = __builtin_amdgcn_readfirstlane(t.row1);
    } else {
        band_order(lid, nm, ntn, mt, c.nt);
        c.group = 0;
        c.row0 = mt * tile_m;
        c.row1 = min(c.row0 + tile_m, g.M);
    }
    return true;
}

__device__ __forceinline__ int64_t a_row_of(const GemmArgs& g, int r) {
    return g.a_map ? (int64_t)(g.a_map[r] / g.a_div) : (int64_t)r;
}

// s_waitcnt with only a vector-memory count (gfx9 encoding: vmcnt[3:0] in
// bits 3:0, vmcnt[5:4] in bits 15:14; expcnt and lgkmcnt left at "no wait").
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
    static_assert(N >= 0 && N < 64, "vmcnt range");
    __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
}

// The same with lgkmcnt(0) as well.
template <int N>
__device__ __forceinline__ void wait_vmcnt_lgkm0() {
    static_assert(N >= 0 && N < 64, "vmcnt range");
    __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4));
}


// s_waitcnt lgkmcnt(0) alone (vmcnt and expcnt left at "no wait").
__device__ __forceinline__ void wait_lgkm0() {
    __builtin_amdgcn_s_waitcnt(15 | (3 << 14) | (7 << 4));
}

__device__ __forceinline__ uint32_t bf16x2_bits(bf16x2_t v) {
    return __builtin_bit_cast(uint32_t, v);
}

// Eight OCP e4m3 codes (code 0 in the low byte of lo) as eight bf16 values.
// e4m3 keeps 3 mantissa bits and exponents 2^-9 .. 2^8, so every finite code
// is exact in bf16.  v_cvt_scalef32_pk_bf16_fp8 with a unit scale converts
// two codes (bytes 0-1, or 2-3 with the high select) in one instruction;
// checked against all 256 codes, the two NaN codes included.
__device__ __forceinline__ u32x4_t fp8x8_to_bf16x8(uint32_t lo, uint32_t hi) {
    u32x4_t r;
    r[0] = bf16x2_bits(__builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(lo, 1.0f, false));
    r[1] = bf16x2_bits(__builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(lo, 1.0f, true));
    r[2] = bf16x2_bits(__builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(hi, 1.0f, false));
    r[3] = bf16x2_bits(__builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(hi, 1.0f, true));
    return r;
}

// The fp32 that carries an E8M0 block exponent e into the scaled
// conversions: they use only the exponent field of their fp32 scale
// (checked: a scale of 3.0 multiplies by 2), so e << 23 stands for 2^(e-127).
// Codes 1 .. 254; 0 and the NaN code 255 are outside what the kernels handle.
__device__ __forceinline__ float e8m0_scale(uint32_t e) { return __uint_as_float(e << 23); }

// Eight OCP E2M1 codes (code 0 in the low nibble of byte 0) times the block
// scale as eight bf16 values.  An E2M1 value (at most 1.5 * 2^2, one mantissa
// bit) times a power of two is exact in bf16 for block exponents the weights
// use; v_cvt_scalef32_pk_bf16_fp4 converts the two codes of byte j (low
// nibble into the low half), checked against all 256 bytes and byte selects.
__device__ __forceinline__ u32x4_t fp4x8_to_bf16x8(uint32_t codes, float scale) {
    u32x4_t r;
    r[0] = bf16x2_bits(__builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(codes, scale, 0));
    r[1] = bf16x2_bits(__builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(codes, scale, 1));
    r[2] = bf16x2_bits(__builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(codes, scale, 2));
    r[3] = bf16x2_bits(__builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(codes, scale, 3));
    return r;
}

}  // namespace tiles
}  // namespace moe
