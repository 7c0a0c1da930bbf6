// jf_group.h -- the "group of four blocks" mapping shared by the INT8 -> INT8
// elementwise and row kernels (GELU backward, residual add, LayerNorm).
//
// A wavefront covers four horizontally adjacent 32x32 blocks (a 32 x 128
// byte tile).  Lane l holds rows 8i + l/8 (i = 0..3) and bytes 16(l%8) ..
// 16(l%8)+15 of each row, i.e. part of block (l%8)/2; every 16-byte load and
// store of the wavefront spans eight whole 128-byte rows.
#pragma once

#include "jf_device.h"

namespace jf {

constexpr int kGroupBlocks = 4;

// Maximum over the 16 lanes holding each block (lanes 8r + 2b + e), in every
// lane for its own block: DPP over lane bits 0 and 3 within each row of 16
// lanes, then the gfx950 row-swapping permutes over lane bits 5 and 4.
// v >= 0, whose IEEE order is the unsigned order of the bits.  Lanes 0, 2, 4
// and 6 hold blocks 0..3.
__device__ __forceinline__ float group_own_block_max(float v) {
    uint32_t u = __float_as_uint(v);
    u = max(u, dpp<kDppXor1>(u));
    u = max(u, dpp<kDppRowRor8>(u));
    const auto h = __builtin_amdgcn_permlane32_swap(u, u, false, false);   // lanes l and l ^ 32
    u = max(h[0], h[1]);
    const auto r = __builtin_amdgcn_permlane16_swap(u, u, false, false);   // lanes l and l ^ 16
    return __uint_as_float(max(r[0], r[1]));
}

// Codes of the lane's 4 x 16 values y (row-major by i) under scale sc,
// stored as four 16-byte rows at dst + 8 i ld.  A zero scale stores zeros.
__device__ __forceinline__ void store_group_codes(const float (&y)[64], float sc, int8_t *dst, int64_t ld) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        float v[16];
#pragma unroll
        for (int e = 0; e < 16; ++e) v[e] = y[16 * i + e];
        int code[16];
        if (sc != 0.0f) {
            quant_codes(v, sc, code);
        } else {
#pragma unroll
            for (int e = 0; e < 16; ++e) code[e] = 0;
        }
        st_stream(reinterpret_cast<u32x4 *>(dst + 8 * i * ld),
                  u32x4{pack4(code[0], code[1], code[2], code[3]), pack4(code[4], code[5], code[6], code[7]),
                        pack4(code[8], code[9], code[10], code[11]), pack4(code[12], code[13], code[14], code[15])});
    }
}

}  // namespace jf
