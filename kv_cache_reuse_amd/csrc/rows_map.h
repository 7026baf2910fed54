// Lane maps of natural-layout (row) KV tiles inside one wave, used by the
// row variants of the step kernels (match.h) and by the host checks.
//
// A row tile is 16 rows of D elements, contiguous, and a wave loads it in
// 1 KiB loads: lane l of load j holds 16-byte piece g = 64 j + l of the
// tile, which is piece g mod PR of row g / PR (PR = D sizeof(T) / 16 pieces
// per row).  The wave writes the pieces, as loaded, into LDS rows RS
// elements apart (RS = D + the pad below) and reads them back in the
// operand order of the library's tiles:
//  - keys: lane (lg, c) = (l / 16, l mod 16) takes piece 4 j + lg of row c
//    as its register j;
//  - bf16 values, with gfx950's transposing LDS read (ds_read_b64_tr_b16):
//    in each block of 16 lanes, lane 4 e + q supplies the address of 4
//    consecutive elements and lane 4 q + r receives element r of the
//    addresses of lanes 4 e + q, e = 0 .. 3, as its elements 0 .. 3 (read
//    off a probe that loads element indices).  A lane that points at token
//    tr16_row(l), dims 16 k + tr16_col(l) .. + 3 hands lane (lg, c) tokens
//    4 lg .. 4 lg + 3 of dim 16 k + c;
//  - fp32 values: lane (lg, c) reads tokens 4 lg .. 4 lg + 3 of dim 16 i + c
//    one by one.
#pragma once

#include <hip/hip_runtime.h>

namespace mac {

constexpr int kRowsPadBf16 = 8;   // bf16 LDS row: D + 8 elements (16-byte aligned)
constexpr int kRowsPadF32 = 4;    // fp32 LDS row: D + 4 floats

__host__ __device__ constexpr int rows_load_row(int j, int lane, int pr) { return (64 * j + lane) / pr; }
__host__ __device__ constexpr int rows_load_piece(int j, int lane, int pr) { return (64 * j + lane) % pr; }
__host__ __device__ constexpr int rows_key_row(int lane) { return lane % 16; }
__host__ __device__ constexpr int rows_key_piece(int j, int lane) { return 4 * j + lane / 16; }
__host__ __device__ constexpr int tr16_row(int lane) { return 4 * (lane / 16) + (lane % 16) / 4; }
__host__ __device__ constexpr int tr16_col(int lane) { return 4 * (lane % 4); }

}  // namespace mac
