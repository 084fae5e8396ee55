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
typedef __attribute__((address_space(3))) void lds_void;
typedef __attribute__((address_space(1))) void glb_void;

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

// LDS tiles are addressed through address_space(3) pointers so that no
// generic-to-local conversion is emitted per access.
typedef const __attribute__((address_space(3))) char lds_cchar;

SAS_DEV lds_char* lds_ptr(char* generic_smem) { return (lds_char*)generic_smem; }

// Integer LDS byte addresses: the backend folds "address + constant" into the
// 16-bit offset field of the DS instruction, so a per-lane base plus
// compile-time tile/chunk offsets costs no VALU per read.
// LDS byte addresses are below 2^18; the mask lets the compiler prove the sign
// bit is clear, which DS offset folding requires.
constexpr uint32_t kLdsAddrMask = (1u << 18) - 1;
SAS_DEV uint32_t lds_addr(lds_cchar* p) {
  return uint32_t(reinterpret_cast<uintptr_t>(p)) & kLdsAddrMask;
}
SAS_DEV bf16x8 lds_read16_at(uint32_t a) {
  return *reinterpret_cast<const __attribute__((address_space(3))) bf16x8*>(uintptr_t(a));
}
SAS_DEV bf16x4 lds_read_tr_at(uint32_t a) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4bf16(
      reinterpret_cast<__attribute__((address_space(3))) bf16x4*>(uintptr_t(a)));
}
SAS_DEV bf16x8 tr_pair_at(uint32_t a0, uint32_t a1) {
  const bf16x4 a = lds_read_tr_at(a0);
  const bf16x4 b = lds_read_tr_at(a1);
  return __builtin_shufflevector(a, b, 0, 1, 2, 3, 4, 5, 6, 7);
}

SAS_DEV bf16x8 lds_read16(lds_cchar* base, int off) {
  return *reinterpret_cast<const __attribute__((address_space(3))) bf16x8*>(base + off);
}

SAS_DEV bf16x4 lds_read_tr(lds_cchar* base, int off) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4bf16(
      (__attribute__((address_space(3))) bf16x4*)(base + off));
}

// Transposed operand of a row-major [64 keys][D] tile: 8 keys x one column per
// lane, keys ordered as the S^T accumulator rows of a 32x32 MFMA tile.
// kbase: first key of the 16-key chunk; col0: first column of the 32-column
// tile.  Lane l gets keys kbase + 4*(l/32) + {0..3} and kbase + 8 + 4*(l/32) +
// {0..3} of column col0 + l%32.
template <int D>
SAS_DEV bf16x8 tr_operand(lds_cchar* tile, int kbase, int col0, int lane) {
  const int i = lane & 15, hh = lane >> 5, dh = (lane >> 4) & 1;
  const int col = col0 + dh * 16 + (i & 3) * 4;
  const int r0 = kbase + 4 * hh + (i >> 2);
  const int r1 = r0 + 8;
  const int sub = (i & 1) << 3;
  const bf16x4 a = lds_read_tr(tile, tile_off<D>(r0, col >> 3) + sub);
  const bf16x4 b = lds_read_tr(tile, tile_off<D>(r1, col >> 3) + sub);
  return __builtin_shufflevector(a, b, 0, 1, 2, 3, 4, 5, 6, 7);
}

// ---------------------------------------------------------------- LDS DMA ring
// GLOBAL_LOAD_LDS_DWORDX4 (checked on the device): lane l's 16 bytes land at
// LDS address base + 16*l (base is wave-uniform); inactive lanes write nothing.
// The loads count in vmcnt like any vector load but need no registers, so a
// workgroup can keep several tiles in flight.
SAS_DEV void dma16(const void* g, lds_char* l) {
  __builtin_amdgcn_global_load_lds((glb_void*)g, (lds_void*)l, 16, 0, 0);
}

// Per-lane byte offsets, inside a 1 KB slice of a swizzled 64 x D tile, of
// the chunk lane `lane` moves, for tiles whose rows are contiguous in global
// memory (row stride D elements) written to LDS in the swizzled layout: each
// lane fetches the logical chunk that belongs at its physical slot.  The
// swizzle of a slice's rows depends on the slice index mod 4 only, so slice
// first + u of a tile at global address g is lane-wise
// g + 1024*(first + u) + pat[u % 4].
template <int D>
SAS_DEV void dma_lane_pattern(int lane, int first, uint32_t (&pat)[4]) {
  constexpr int CPR = D / 8;
  constexpr int RPI = 64 / CPR;
#pragma unroll
  for (int t = 0; t < 4; ++t) {
    const int r = (first + t) * RPI + lane / CPR;
    const int c = (lane % CPR) ^ swz<D>(r);
    pat[t] = uint32_t((lane / CPR) * D * 2 + c * 16);
  }
}

// Hide a value from the optimiser (so "base + lane offset" stays one register
// and only the small per-access constant goes to the DS offset field).
SAS_DEV uint32_t opaque(uint32_t x) {
  asm volatile("" : "+v"(x));
  return x;
}

// A wave-uniform global address, held in SGPRs: a DMA from it plus a 32-bit
// lane offset issues in the scalar-base + vector-offset form, with no
// per-lane 64-bit address arithmetic.  Only for addresses every lane of the
// wave shares.
SAS_DEV const char* uniform_ptr(const void* p) {
  const uint64_t a = reinterpret_cast<uint64_t>(p);
  const uint32_t lo = __builtin_amdgcn_readfirstlane(uint32_t(a));
  const uint32_t hi = __builtin_amdgcn_readfirstlane(uint32_t(a >> 32));
  return reinterpret_cast<const char*>((uint64_t(hi) << 32) | lo);
}

// A contiguous run of N slices, first .. first+N-1, of the tile at gtile
// (wave-uniform) into the LDS tile ltile.
template <int N>
SAS_DEV void dma_slices(const void* gtile, lds_char* ltile, int first, const uint32_t (&pat)[4]) {
  const char* g = reinterpret_cast<const char*>(gtile) + first * 1024;
  lds_char* l = ltile + first * 1024;
#pragma unroll
  for (int u = 0; u < N; ++u) dma16(uniform_ptr(g + u * 1024) + opaque(pat[u & 3]), l + u * 1024);
}

// Wait until at most N of this wave's vector memory operations are
// outstanding and all its LDS operations are done, then barrier.  Raw
// s_barrier: __syncthreads() adds a release fence that waits for every
// outstanding load (vmcnt(0)) and would drain the DMA ring.  The empty asm
// statements keep the compiler from moving memory operations across.
template <int N>
SAS_DEV void vm_wait_barrier() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | (7 << 4) | (0 << 8) | ((N >> 4) << 14));
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}


// ---------------------------------------------------------------- LDS ring buffers
// Every ring stage (and tile kind) is its own __shared__ variable, reached
// with a compile-time stage index.  The compiler then knows which buffer an
// LDS read touches and which buffers in-flight DMA writes, and waits only for
// the DMA that filled the stage being read (with one LDS variable and a
// runtime stage index it drains every outstanding load before each
// transposed read).
template <int TAG, int ST, int BYTES>
SAS_DEV lds_char* stage_buf() {
  __shared__ __attribute__((aligned(16))) char buf[BYTES];
  return (lds_char*)buf;
}

// Per-lane byte offset kept in a register: hidden from re-association and
// masked so that the compiler can prove it non-negative, which lets every
// "buffer + offset + constant" access fold the constant into the DS
// instruction's offset field.
SAS_DEV uint32_t lane_off(int raw) { return opaque(uint32_t(raw)) & kLdsAddrMask; }

SAS_DEV bf16x8 ld16(lds_cchar* base, uint32_t off) {
  return *reinterpret_cast<const __attribute__((address_space(3))) bf16x8*>(base + off);
}
SAS_DEV bf16x4 ldtr(lds_cchar* base, uint32_t off) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4bf16(
      (__attribute__((address_space(3))) bf16x4*)(base + off));
}
SAS_DEV bf16x8 ldtr_pair(lds_cchar* base, uint32_t off0, uint32_t off1) {
  const bf16x4 a = ldtr(base, off0);
  const bf16x4 b = ldtr(base, off1);
  return __builtin_shufflevector(a, b, 0, 1, 2, 3, 4, 5, 6, 7);
}

constexpr int kFwdStages = 3;   // K/V tile ring depth of the forward
constexpr int kDqStages = 2;    // K/V tile ring depth of the dq pass (register-bound)
constexpr int kKvStages = 4;    // Q/dO tile ring depth of the key-block-outer kernel

// Host: a query-head group of G heads is covered by launches of 4-, 2- and
// 1-head workgroups (so the DMA slices split evenly over the waves).
struct HeadChunks {
  int gc, h_off, count;  // heads per workgroup, first head, chunks in launch
};
inline int head_chunk_list(int G, HeadChunks* out) {
  int nlist = 0, h = 0;
  for (int gc = 4; gc >= 1; gc >>= 1) {
    const int c = (G - h) / gc;
    if (c > 0) {
      out[nlist++] = HeadChunks{gc, h, c};
      h += c * gc;
    }
  }
  return nlist;
}
struct HeadChunkSet {
  HeadChunks v[3];
  int nv;
  const HeadChunks* begin() const { return v; }
  const HeadChunks* end() const { return v + nv; }
};
inline HeadChunkSet head_chunks(int G) {
  HeadChunkSet s{};
  s.nv = head_chunk_list(G, s.v);
  return s;
}

template <class K>
inline void allow_lds(K kernel, size_t bytes) {
  if (bytes > 65536)
    (void)hipFuncSetAttribute(reinterpret_cast<const void*>(kernel),
                              hipFuncAttributeMaxDynamicSharedMemorySize, int(bytes));
}

// Transposed operand read with precomputed per-lane offsets (see tr_offsets).
SAS_DEV bf16x8 tr_operand_at(lds_cchar* tile, int off0, int off1) {
  const bf16x4 a = lds_read_tr(tile, off0);
  const bf16x4 b = lds_read_tr(tile, off1);
  return __builtin_shufflevector(a, b, 0, 1, 2, 3, 4, 5, 6, 7);
}

// Per-lane byte offsets of the two DS_READ_B64_TR_B16 reads of tr_operand for a
// 16-row chunk starting at row 0 and the 32-column tile dt.  For a chunk that
// starts at row kbase (a multiple of 16) the offsets are kbase*2*D larger: the
// swizzle depends on row % 16 only.
template <int D>
SAS_DEV void tr_offsets(int lane, int (&off)[D / 32][2]) {
  const int i = lane & 15, hh = lane >> 5, dh = (lane >> 4) & 1;
#pragma unroll
  for (int dt = 0; dt < D / 32; ++dt)
#pragma unroll
    for (int w = 0; w < 2; ++w) {
      const int r = 4 * hh + (i >> 2) + 8 * w;
      const int col = dt * 32 + dh * 16 + (i & 3) * 4;
      off[dt][w] = (tile_off<D>(r, col >> 3) + ((i & 1) << 3)) & int(kLdsAddrMask);
    }
}

// Per-lane byte offsets of the 16-byte row reads of rows r0 + (lane % 32),
// chunks 2c + lane/32 (c < D/16), for r0 a multiple of 16.
template <int D>
SAS_DEV void row_offsets(int lane, int (&off)[D / 16]) {
  const int lr = lane & 31, hh = lane >> 5;
#pragma unroll
  for (int c = 0; c < D / 16; ++c) off[c] = tile_off<D>(lr, 2 * c + hh) & int(kLdsAddrMask);
}


typedef __attribute__((ext_vector_type(2))) __bf16 bf16x2;

// Sum of the 8 bf16 values (accumulated in float32) added to acc.
SAS_DEV float sum_bf16x8(const bf16x8& v, float acc) {
  const bf16x2 one = {(__bf16)1.0f, (__bf16)1.0f};
  acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_shufflevector(v, v, 0, 1), one, acc, false);
  acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_shufflevector(v, v, 2, 3), one, acc, false);
  acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_shufflevector(v, v, 4, 5), one, acc, false);
  acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_shufflevector(v, v, 6, 7), one, acc, false);
  return acc;
}

SAS_DEV bf16x8 pack_bf16x8(const float* x) {
  bf16x8 r;
#pragma unroll
  for (int e = 0; e < 8; ++e) r[e] = (__bf16)x[e];
  return r;
}

}  // namespace sas
