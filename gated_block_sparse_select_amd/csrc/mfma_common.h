// bf16 matrix-core helpers for gfx950 (CDNA4), wave64.
//
// Operand layouts of V_MFMA_F32_32X32X16_BF16 (checked on the device):
//   A (32x16, M x K): lane l holds A[m = l%32][k = 8*(l/32) + e], e = 0..7
//   B (16x32, K x N): lane l holds B[k = 8*(l/32) + e][n = l%32]
//   C (32x32):        lane l, register j holds C[m = 8*(j/4) + 4*(l/32) + j%4][n = l%32]
// DS_READ_B64_TR_B16 (checked on the device): inside each group of 16 lanes,
// lane i receives element (i%4) of the 4-element rows addressed by lanes
// i/4, 4 + i/4, 8 + i/4 and 12 + i/4 (in that order).
//
// 64 x D bf16 tiles live row-major in LDS with the 16-byte chunks of each row
// XOR-swizzled per row (swz below).
#pragma once

#include "common.h"

namespace sas {

typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8;
typedef __attribute__((ext_vector_type(4))) __bf16 bf16x4;
typedef __attribute__((ext_vector_type(16))) float f32x16;
typedef __attribute__((address_space(3))) char lds_char;

SAS_DEV f32x16 mfma32(const bf16x8& a, const bf16x8& b, const f32x16& c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

// Chunk swizzle of a 64 x D tile.  Physical chunk = logical chunk ^ f(row) with
//   f(row) = base[row & 3] ^ ((row >> 2) & 3),
//   base = {0, 6, 12, 10} (D = 128, 16 chunks per row) or {0, 2, 4, 6} (D = 64).
// Within 4 consecutive rows the base values differ in bits 1-2 and in bits 2-3,
// so the 8 (16) chunks touched by a transposed read of 16 (32) lanes fall in
// distinct banks; the (row >> 2) term spreads 8 / 16 consecutive rows of a row
// read over all chunk positions.  One swizzle serves both read kinds, so a tile
// can be read row-wise and transposed.
template <int D>
SAS_DEV int swz(int row) {
  const int base = D == 128 ? ((0xAC60 >> ((row & 3) * 4)) & 15) : ((row & 3) * 2);
  return base ^ ((row >> 2) & 3);
}

// Byte offset of logical 16-byte chunk `ch` of row `row` in a swizzled tile.
template <int D>
SAS_DEV int tile_off(int row, int ch) {
  return row * (D * 2) + ((ch ^ swz<D>(row)) << 4);
}

SAS_DEV bf16x8 lds_read16(const char* base, int off) {
  return *reinterpret_cast<const bf16x8*>(base + off);
}

SAS_DEV bf16x4 lds_read_tr(const char* base, int off) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4bf16(
      (__attribute__((address_space(3))) bf16x4*)((lds_char*)base + off));
}

// Transposed operand of a row-major [64 keys][D] tile: 8 keys x one column per
// lane, keys ordered as the S^T accumulator rows of a 32x32 MFMA tile.
// kbase: first key of the 16-key chunk; col0: first column of the 32-column
// tile.  Lane l gets keys kbase + 4*(l/32) + {0..3} and kbase + 8 + 4*(l/32) +
// {0..3} of column col0 + l%32.
template <int D>
SAS_DEV bf16x8 tr_operand(const char* tile, int kbase, int col0, int lane) {
  const int i = lane & 15, hh = lane >> 5, dh = (lane >> 4) & 1;
  const int col = col0 + dh * 16 + (i & 3) * 4;
  const int r0 = kbase + 4 * hh + (i >> 2);
  const int r1 = r0 + 8;
  const int sub = (i & 1) << 3;
  const bf16x4 a = lds_read_tr(tile, tile_off<D>(r0, col >> 3) + sub);
  const bf16x4 b = lds_read_tr(tile, tile_off<D>(r1, col >> 3) + sub);
  return __builtin_shufflevector(a, b, 0, 1, 2, 3, 4, 5, 6, 7);
}

SAS_DEV bf16x8 pack_bf16x8(const float* x) {
  bf16x8 r;
#pragma unroll
  for (int e = 0; e < 8; ++e) r[e] = (__bf16)x[e];
  return r;
}

}  // namespace sas
