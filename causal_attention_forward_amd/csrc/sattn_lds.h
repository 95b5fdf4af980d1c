// LDS layout of the 64 x 64 binary16 tiles staged unpadded by the backward
// and the split-key forward, the gfx950 transpose read that turns such a
// tile into a matrix-core operand of its transpose, and the direct-to-LDS
// loads that stage them.
#ifndef SATTN_LDS_H
#define SATTN_LDS_H

#include <hip/hip_runtime.h>

namespace sattn_lds {

typedef _Float16 half_t;
typedef _Float16 half4 __attribute__((ext_vector_type(4)));
typedef _Float16 half8 __attribute__((ext_vector_type(8)));
typedef short short4v __attribute__((ext_vector_type(4)));

constexpr int kRowHalfs = 64;  // an LDS row: 64 values in eight 16-byte chunks

// ds_read_b64_tr_b16 at p: within each 16-lane group, lane 4a + b supplies
// the address of row a, columns 4b'..4b'+3 of a block, and lane t receives
// rows 0..3 of the column that lanes 4(t/4)'s supplier pointed at, offset t%4.
__device__ __forceinline__ half4 lds_tr4(const half_t* p) {
  typedef __attribute__((address_space(3))) short4v lds_short4;
  const short4v v = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_short4*)(const_cast<half_t*>(p)));
  return __builtin_bit_cast(half4, v);
}

// Tiles keep 64-value rows unpadded and place 16-byte chunk c of row r at
// chunk c ^ swz(r), swz(r) = the three bits of (r/2) % 8 reversed.  Sixteen
// lanes reading one chunk of 16 consecutive rows (the natural operand read)
// then hit all 64 banks once, and so do 32 lanes of a transpose read (four
// rows, four chunks each): rows r and r+2 land in opposite halves of the row
// and odd rows in the other 32 banks.  A row pad cannot do both.  swz
// depends on r only through (r/2) % 8, so an offset of 16 rows keeps it.
__device__ __forceinline__ int swz(int r) {
  const int v = (r >> 1) & 7;
  return ((v & 1) << 2) | (v & 2) | (v >> 2);
}

// Offset (halfs) of 16-byte chunk c of row r in a swizzled tile.
__device__ __forceinline__ int chunk_offset(int r, int c) { return r * kRowHalfs + ((c ^ swz(r)) << 3); }

// Operand whose lane l holds X[m][k0 + 8(l/32) .. +7] for a tile stored
// k-major in LDS (X[m][k] at row k, column m): two transpose reads, rows
// k .. k+3 at lo and k+4 .. k+7 at hi (offsets include the lane's own part).
__device__ __forceinline__ half8 tr8(const half_t* base, int lo, int hi) {
  const half4 a = lds_tr4(base + lo), b = lds_tr4(base + hi);
  return half8{a[0], a[1], a[2], a[3], b[0], b[1], b[2], b[3]};
}

// A lane's tr8 offset (halfs) over a k-major tile for operand rows m in
// 32 mh .. 32 mh + 31 and the read of rows 4 hi .. (hi = 0, 1): row
// 8(l/32) + (l%16)/4 + 4 hi, column 32 mh + 16((l/16)%2) + 4 c(l%4), where c
// is the identity (the operand's row m is l%32) or swaps the two bits of l%4
// (its row m is krow(l%32), bits 2 and 3 of the row swapped).
__device__ __forceinline__ int tr_offset(int lane, bool permuted, int mh, int hi) {
  const int b = lane & 3;
  const int cb = permuted ? (((b & 1) << 1) | (b >> 1)) : b;
  const int row = 8 * (lane >> 5) + ((lane & 15) >> 2) + 4 * hi;
  const int col = 32 * mh + 16 * ((lane >> 4) & 1) + 4 * cb;
  return chunk_offset(row, col >> 3) + (col & 7);
}

typedef int int4v __attribute__((ext_vector_type(4)));

// Direct-to-LDS loads (buffer_load ... lds): lane l's 16 (or 4) bytes at byte
// offset voff of the buffer that rsrc describes land at LDS byte
// lds + 16 l (or 4 l); lds goes in M0, with one wait state before the load
// reads it.  Offsets past the buffer's range read zeros.  The compiler does
// not see these loads: callers wait for them with s_waitcnt vmcnt.
__device__ __forceinline__ void lds_load16(const int4v& rsrc, unsigned lds, unsigned voff) {
  asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tbuffer_load_dwordx4 %1, %2, 0 offen lds"
               :
               : "s"(lds), "v"(voff), "s"(rsrc)
               : "memory", "m0");
}
__device__ __forceinline__ void lds_load4(const int4v& rsrc, unsigned lds, unsigned voff) {
  asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tbuffer_load_dword %1, %2, 0 offen lds"
               :
               : "s"(lds), "v"(voff), "s"(rsrc)
               : "memory", "m0");
}

// A raw buffer descriptor (32-bit data format, no stride) as an SGPR quad.
__device__ __forceinline__ int4v raw_desc(const void* base, unsigned bytes) {
  const unsigned long long a = (unsigned long long)base;
  return int4v{__builtin_amdgcn_readfirstlane((int)(unsigned)a),
               __builtin_amdgcn_readfirstlane((int)(unsigned)(a >> 32) & 0xFFFF),
               __builtin_amdgcn_readfirstlane((int)bytes), 0x00020000};
}

// The LDS byte address of p.
__device__ __forceinline__ unsigned lds_addr(const void* p) {
  return (unsigned)(size_t)(__attribute__((address_space(3))) const char*)p;
}

// The s_waitcnt operand that waits until at most n vector memory operations
// are outstanding and for nothing else.
constexpr int vmcnt_only(int n) { return (n & 15) | ((n >> 4) << 14) | 0x0F70; }

}  // namespace sattn_lds

#endif  // SATTN_LDS_H
