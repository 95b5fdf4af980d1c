// The causal streaming-attention forward for problems too small to fill the
// chip (few query blocks per K/V head): the key range of each 32-row query
// block is split over the four waves of a workgroup, and the four partial
// results are merged at the end by the rule the method uses between tiles.
//
// Method (StreamingAttentionSM86 page, header comment and tile body of the
// forward realization): per 64-key tile, S^T = K Q^T on the matrix cores,
// base-2 scores t = S c, a running row maximum m, row sum l and weighted sum
// O folded by the merge rule for normalised weighted sums (a new maximum m'
// scales l and O by 2^(m - m')), P = 2^(t - m') rounded to binary16 for its
// product with V, sums in binary32; the epilogue writes O / l (binary16,
// token-major) and m + log2 l.  Where V^T can be staged through LDS
// (T % 8 == 0 and the grid fits the chip at once) the reference is moved
// lazily, as in the eight-wave kernel: each wave takes its first tile's exact
// maximum and keeps it while every partial row sum stays within (0, 2^8]
// (the merge rule holds for any reference, so this changes only rounding);
// elsewhere every tile moves it, as the page's tile body does.  The V^T and
// V-rows entries make the same choice, so they give the same bits.
//
// gfx950 design:
//  * Workgroup = four waves on one 32-row query block of one head; wave w
//    takes key tiles w, w + 4, w + 8, ... up to the block's diagonal, so a
//    block's key range is walked four times faster than by one wave.
//  * Each wave stages its own tiles in a private LDS region, so the loop
//    has no barrier: a tile's K rows and V^T rows (or V rows) are read with
//    fully coalesced 16-byte loads (eight whole 128-byte lines per
//    instruction; rows and keys past T read as zeros through the buffer
//    range checks) and stored swizzled so that the operand reads hit every
//    bank once.  Given V as rows, the V^T operand comes from transpose reads
//    of the V-rows tile.  (Operands loaded straight from global memory, as
//    16-byte pieces of 32 different lines per instruction, left the CU's
//    load path the bottleneck.)
//  * Two ways of staging.  When the grid fits the chip in one wave of
//    workgroups (one per CU) and V comes in whole 16-byte chunks (V rows, or
//    V^T with T % 8 == 0), the loads go straight into LDS (buffer_load ...
//    lds) and each wave has two buffers, so the tile four further along is
//    in flight while one is computed; the loads are issued from inline
//    assembly and waited for with explicit vmcnt counts.  Otherwise two
//    workgroups share a CU and each wave holds the next tile in registers
//    while computing the current one.
//  * S^T = K Q^T and O^T = V^T P^T on v_mfma_f32_32x32x16_f16 (a lane owns one
//    query and 16 keys, so a row's max and sum are in-lane plus one exchange
//    with the lane 32 away); K rows are permuted so each lane's 8 keys per
//    16-key slice of P^T are consecutive (one 16-byte V^T read per operand).
//  * The merge: waves 1..3 leave m, l and O^T in their LDS regions; wave 0 forms
//    M = max m_w, l = sum l_w 2^(m_w - M), O = sum O_w 2^(m_w - M) and writes
//    O / l and M + log2 l.
#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>

#include "sattn.h"
#include "sattn_internal.h"
#include "sattn_lds.h"

namespace {

typedef _Float16 half_t;
typedef _Float16 half4 __attribute__((ext_vector_type(4)));
typedef _Float16 half8 __attribute__((ext_vector_type(8)));
typedef float float4v __attribute__((ext_vector_type(4)));
typedef float float16v __attribute__((ext_vector_type(16)));
typedef int int4v __attribute__((ext_vector_type(4)));

using sattn_lds::chunk_offset;
using sattn_lds::lds_addr;
using sattn_lds::lds_load16;
using sattn_lds::raw_desc;
using sattn_lds::tr8;
using sattn_lds::tr_offset;

constexpr int kD = SATTN_HEAD_DIM;
constexpr int kWaves = 4;
constexpr int kXcds = 8;
constexpr int kCus = 256;  // compute units per MI355X
constexpr int kTileHalfs = 64 * sattn_lds::kRowHalfs;  // one staged 64 x 64 tile
constexpr int kBufferWord3 = 0x00020000;               // raw buffer, 32-bit data format
constexpr int kOutOfRange = 0x7FFFFFF0;                // a buffer offset past every range
constexpr int kLdsDone = 0xC07F;                       // s_waitcnt lgkmcnt(0) only
constexpr int kVmcnt16 = sattn_lds::vmcnt_only(16);   // s_waitcnt vmcnt(16) only
constexpr int kVmcnt0 = sattn_lds::vmcnt_only(0);     // s_waitcnt vmcnt(0) only

__device__ __forceinline__ float16v mfma(half8 a, half8 b, float16v c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ float xlane(float x, int addr) {
  return __builtin_bit_cast(float, __builtin_amdgcn_ds_bpermute(addr, __builtin_bit_cast(int, x)));
}

// K row loaded by operand row m of S^T = K Q^T: accumulator element i of lane
// (n, g) is then key 16*(i/8) + 8g + i%8 of the 32-key block.
__device__ __forceinline__ int krow(int m) {
  const int a = m >> 3, e = (m >> 2) & 1, b = m & 3;
  return 16 * (a >> 1) + 8 * e + 4 * (a & 1) + b;
}

__device__ __forceinline__ half8 ld8(const half_t* p) { return *reinterpret_cast<const half8*>(p); }

// a compiler fence after an explicit wait, so no LDS read moves above it
__device__ __forceinline__ void wait_vm(bool keep16) {
  if (keep16) __builtin_amdgcn_s_waitcnt(kVmcnt16);
  else __builtin_amdgcn_s_waitcnt(kVmcnt0);
  asm volatile("" ::: "memory");
}

template <bool VT_VEC, bool VROWS, bool DMA, bool LAZY>
__global__ void __launch_bounds__(64 * kWaves, DMA ? 1 : 2)
sattn_fwd_split_kernel(const half_t* __restrict__ Q, const half_t* __restrict__ K,
                       const half_t* __restrict__ Vt, half_t* __restrict__ O,
                       float* __restrict__ L, float c, int T, int Hq, int G, int nBlocks,
                       int nPairs, int pairsPerXcd) {
  // Wave w's region: a K tile and a V^T (or V-rows) tile; with DMA a second
  // such pair and its 32 Q rows.  After the key loop it holds the wave's
  // partial (O^T, m, l) for the merge.
  static_assert(!DMA || VT_VEC || VROWS, "LDS loads need whole 16-byte V chunks");
  static_assert(!LAZY || DMA, "the lazy reference's slow path needs the registers LDS staging frees");
  constexpr int kRegionHalfs = DMA ? 4 * kTileHalfs + 32 * sattn_lds::kRowHalfs : 2 * kTileHalfs;
  __shared__ __attribute__((aligned(16))) half_t lds[kWaves * kRegionHalfs];

  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lane = tid & 63;
  const int n = lane & 31;
  const int g = lane >> 5;

  // Query blocks are paired, heavy n-1-j with light j (every pair carries
  // about the same causal work), and pairs are numbered K/V head first, then
  // j, then the group's query heads.  Workgroups are dealt to the XCDs
  // round-robin; XCD x takes the contiguous run of pairs x*pairsPerXcd ..,
  // its first pairsPerXcd workgroups their heavy blocks (heaviest first) and
  // the next pairsPerXcd the light blocks of the same pairs, so the XCDs
  // carry equal work and, where two workgroups share a CU, a CU's two
  // workgroups are one pair.  The grid is padded to whole runs; padding and
  // the missing partner of an odd middle block exit at once.
  const int xcd = blockIdx.x % kXcds, pos = blockIdx.x / kXcds;
  const bool light = pos >= pairsPerXcd;
  const int pair = xcd * pairsPerXcd + (light ? pos - pairsPerXcd : pos);
  if (pair >= nPairs) return;
  const int perKv = ((nBlocks + 1) / 2) * G;
  const int kv = pair / perKv;
  const int j = (pair - kv * perKv) / G;
  const int h = kv * G + (pair - kv * perKv) % G;
  const int blk = light ? j : nBlocks - 1 - j;
  if (light && j >= nBlocks - 1 - j) return;

  const int row = 32 * blk + n;
  const int need = min(T - 1, 32 * blk + 31) / 64 + 1;  // key tiles up to the diagonal

  half_t* const region = lds + wave * kRegionHalfs;
  half8 qf[4];
  if constexpr (!DMA) {
#pragma unroll
    for (int kk = 0; kk < 4; ++kk)
      qf[kk] = row < T ? ld8(Q + ((size_t)h * T + row) * kD + 16 * kk + 8 * g) : half8{};
  }

  // Staging: lane l owns 16-byte chunk l + 64 i (i < 8) of each tile: row
  // l/8 + 8i, chunk l%8.  K (and V rows) tiles are 8 KiB contiguous; a V^T
  // tile is 64 rows of 128 bytes, T values apart.
  half_t* const ktile = region;
  half_t* const vtile = region + kTileHalfs;
  const int sr = lane >> 3, sc = lane & 7;
  const half_t* Vh = Vt + (size_t)kv * kD * T;  // V^T of head kv, or (VROWS) its V rows
  const __amdgpu_buffer_rsrc_t krsrc = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<half_t*>(K + (size_t)kv * T * kD), 0, T * kD * 2, kBufferWord3);
  const __amdgpu_buffer_rsrc_t vrsrc =
      __builtin_amdgcn_make_buffer_rsrc(const_cast<half_t*>(Vh), 0, kD * T * 2, kBufferWord3);
  int4v st[16];  // the next tile: K chunks 0..7, V chunks 8..15
  auto load = [&](int kt) {
    const int key0 = kt * 64;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int r = sr + 8 * i;
      st[i] = __builtin_amdgcn_raw_buffer_load_b128(krsrc, ((key0 + r) * kD + sc * 8) * 2, 0, 0);
      if (VROWS) {  // rows past T read as zeros, like K's
        st[8 + i] = __builtin_amdgcn_raw_buffer_load_b128(vrsrc, ((key0 + r) * kD + sc * 8) * 2, 0, 0);
      } else if (VT_VEC) {  // T % 8 == 0: a chunk lies wholly before or past T
        const int off = key0 + sc * 8 < T ? (r * T + key0 + sc * 8) * 2 : kOutOfRange;
        st[8 + i] = __builtin_amdgcn_raw_buffer_load_b128(vrsrc, off, 0, 0);
      } else {
        const int k0 = key0 + sc * 8;
        half8 x;
#pragma unroll
        for (int e = 0; e < 8; ++e) x[e] = k0 + e < T ? Vh[(size_t)r * T + k0 + e] : (half_t)0;
        st[8 + i] = __builtin_bit_cast(int4v, x);
      }
    }
  };
  auto store = [&]() {
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int off = chunk_offset(sr + 8 * i, sc);
      *reinterpret_cast<int4v*>(ktile + off) = st[i];
      *reinterpret_cast<int4v*>(vtile + off) = st[8 + i];
    }
  };
  // Operand reads: K rows krow(n) (+32) and V^T rows n (+32), chunk 2j + g;
  // with V rows, transpose reads of keys 16 ks .. of the V-rows tile.
  int kOff[4], vOff[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    kOff[j] = chunk_offset(krow(n), 2 * j + g);
    vOff[j] = chunk_offset(n, 2 * j + g);
  }
  int tOff[2][2];
#pragma unroll
  for (int mh = 0; mh < 2; ++mh)
#pragma unroll
    for (int hi = 0; hi < 2; ++hi) tOff[mh][hi] = VROWS ? tr_offset(lane, false, mh, hi) : 0;
  float m = -INFINITY, l = 0.0f;
  float16v o0 = {}, o1 = {};
  const int swapAddr = (lane ^ 32) << 2;
  // one tile: S^T, the mask on the diagonal tile, the new maximum, P, the
  // rescale of l and O, P V
  auto compute = [&](const half_t* kt_lds, const half_t* vt_lds, int kt) {
    const bool first = kt == wave;  // the wave's first tile
    auto vt_operand = [&](int ks, int hf) -> half8 {
      if constexpr (VROWS)
        return tr8(vt_lds + 16 * ks * sattn_lds::kRowHalfs, tOff[hf][0], tOff[hf][1]);
      else
        return ld8(vt_lds + vOff[ks] + 32 * hf * sattn_lds::kRowHalfs);
    };
    float16v s0, s1;
    auto scores = [&]() {  // S^T, masked on the tile crossing the block's diagonal
      s0 = float16v{};
      s1 = float16v{};
#pragma unroll
      for (int kk = 0; kk < 4; ++kk) {
        s0 = mfma(ld8(kt_lds + kOff[kk]), qf[kk], s0);
        s1 = mfma(ld8(kt_lds + kOff[kk] + 32 * sattn_lds::kRowHalfs), qf[kk], s1);
      }
      if (kt == need - 1) {
        const int lim = row - kt * 64 - 8 * g;
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const int k = 16 * (i >> 3) + (i & 7);
          if (k > lim) s0[i] = -INFINITY;
          if (k + 32 > lim) s1[i] = -INFINITY;
        }
      }
    };
    // the reference moved to the tile's maximum (finite: key 64 kt <= row for
    // every row), l and O rescaled to it
    auto exact_reference = [&]() {
      float x = -INFINITY;
#pragma unroll
      for (int i = 0; i < 16; ++i) x = fmaxf(x, fmaxf(s0[i], s1[i]));
      x = fmaxf(x, xlane(x, swapAddr));
      const float m_new = fmaxf(m, x * c);
      const float alpha = __builtin_amdgcn_exp2f(m - m_new);  // 0 when m = -inf
      m = m_new;
      l *= alpha;
      o0 *= alpha;
      o1 *= alpha;
    };
    auto exponentials = [&]() -> float {
      float sum = 0.0f;
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        s0[i] = __builtin_amdgcn_exp2f(fmaf(s0[i], c, -m));
        s1[i] = __builtin_amdgcn_exp2f(fmaf(s1[i], c, -m));
        sum += s0[i] + s1[i];
      }
      return sum;
    };
    scores();
    // Lazy: after the wave's first tile the reference stays put while every
    // lane's partial row sum stays within (0, 2^8]; otherwise the slow path
    // moves it (exactly by a power of two, or to the tile's maximum if a P
    // overflowed).  Eager: every tile moves it.
    if (first || !LAZY) exact_reference();
    float lsum = exponentials();
    if (LAZY && !first && __builtin_amdgcn_ballot_w64(!(lsum <= 256.0f)) != 0) {
      float x = 0.0f;
#pragma unroll
      for (int i = 0; i < 16; ++i) x = fmaxf(x, fmaxf(s0[i], s1[i]));
      const float pmax = fmaxf(x, xlane(x, swapAddr));
      if (__builtin_amdgcn_ballot_w64(!(pmax < INFINITY)) == 0) {
        const int e = pmax > 1.0f ? __builtin_amdgcn_frexp_expf(pmax) : 0;
        const float alpha = __builtin_ldexpf(1.0f, -e);
        m += (float)e;
        l *= alpha;
        o0 *= alpha;
        o1 *= alpha;
        s0 *= alpha;
        s1 *= alpha;
        lsum = 0.0f;
#pragma unroll
        for (int i = 0; i < 16; ++i) lsum += s0[i] + s1[i];
      } else {
        scores();
        exact_reference();
        lsum = exponentials();
      }
    }
    l += lsum;
    half8 p[4];
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      p[0][e] = (half_t)s0[e];
      p[1][e] = (half_t)s0[8 + e];
      p[2][e] = (half_t)s1[e];
      p[3][e] = (half_t)s1[8 + e];
    }
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
      o0 = mfma(vt_operand(ks, 0), p[ks], o0);
      o1 = mfma(vt_operand(ks, 1), p[ks], o1);
    }
  };

  int kt = wave;
  if constexpr (DMA) {
    // Direct-to-LDS staging.  Piece i (1 KiB) of a tile holds its rows 8i ..
    // 8i+7, and lane l's 16 bytes land at row 8i + l/8, chunk slot l%8, the
    // slot of chunk (l%8) ^ swz(row); swz depends on the row only through
    // (row/2) % 8, here on i % 2.
    const int pr = lane >> 3;
    int pc[2];
#pragma unroll
    for (int e = 0; e < 2; ++e) pc[e] = (lane & 7) ^ sattn_lds::swz(8 * e + pr);
    const int4v kdesc = raw_desc(K + (size_t)kv * T * kD, (unsigned)T * kD * 2);
    const int4v vdesc = raw_desc(Vh, (unsigned)kD * T * 2);
    half_t* const kA = region;
    half_t* const vA = region + kTileHalfs;
    half_t* const kB = region + 2 * kTileHalfs;
    half_t* const vB = region + 3 * kTileHalfs;
    half_t* const qrows = region + 4 * kTileHalfs;
    // Sixteen loads per tile.  The wave's earlier reads of the buffer have
    // returned (the products consumed them) before it is refilled.
    auto issue = [&](half_t* kdst, half_t* vdst, int t) {
      __builtin_amdgcn_s_waitcnt(kLdsDone);
      const unsigned key0 = (unsigned)t * 64u;
      const unsigned kl = lds_addr(kdst), vl = lds_addr(vdst);
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const unsigned r = 8u * i + pr, ch = (unsigned)pc[i & 1];
        const unsigned kByte = ((key0 + r) * kD + ch * 8) * 2;  // rows past T: past the range
        lds_load16(kdesc, __builtin_amdgcn_readfirstlane(kl + 1024u * i), kByte);
        unsigned vByte = kByte;  // V rows
        if (!VROWS)  // V^T: chunks at or past T (T % 8 == 0) take an offset past the range
          vByte = key0 + ch * 8 < (unsigned)T ? (r * (unsigned)T + key0 + ch * 8) * 2
                                              : (unsigned)kOutOfRange;
        lds_load16(vdesc, __builtin_amdgcn_readfirstlane(vl + 1024u * i), vByte);
      }
    };
    // Q rows (four pieces, rows past T read as zeros), then tiles kt and
    // kt + 4: loads complete in order, so waiting for all but the last
    // sixteen (or for all, with one tile) covers Q and tile kt.
    {
      const int4v qdesc = raw_desc(Q + (size_t)h * T * kD, (unsigned)T * kD * 2);
      const unsigned ql = lds_addr(qrows);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const unsigned r = 32u * blk + 8u * i + pr;
        lds_load16(qdesc, __builtin_amdgcn_readfirstlane(ql + 1024u * i),
                   (r * kD + (unsigned)pc[i & 1] * 8) * 2);
      }
    }
    if (kt < need) issue(kA, vA, kt);
    if (kt + kWaves < need) issue(kB, vB, kt + kWaves);
    wait_vm(kt + kWaves < need);
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) qf[kk] = ld8(qrows + chunk_offset(n, 2 * kk + g));
    // Tile t computes from one buffer while t + 4 lands in the other; then
    // t + 8 is loaded into the first.  Before computing t, the sixteen loads
    // of t + 4 (issued after t's) may stay outstanding.
    while (kt < need) {
      wait_vm(kt + kWaves < need);
      compute(kA, vA, kt);
      if (kt + 2 * kWaves < need) issue(kA, vA, kt + 2 * kWaves);
      kt += kWaves;
      if (kt >= need) break;
      wait_vm(kt + kWaves < need);
      compute(kB, vB, kt);
      if (kt + 2 * kWaves < need) issue(kB, vB, kt + 2 * kWaves);
      kt += kWaves;
    }
  } else {
    if (kt < need) load(kt);
    while (kt < need) {
      // this wave's own region: its reads of the previous tile were consumed
      // by the products, so the stores may overwrite it
      store();
      __builtin_amdgcn_s_waitcnt(kLdsDone);
      const int kn = kt + kWaves;
      if (kn < need) load(kn);
      compute(ktile, vtile, kt);
      kt = kn;
    }
  }

  // merge the four waves' (m, l, O) of the same 32 rows; l is a partial sum
  // per lane (keys of its half), so the pair's sums are added first
  l += xlane(l, swapAddr);
  // Each wave leaves its O rows (binary32, row-major, 68-float rows), its m
  // and its l in its own region; then wave w merges rows 8w .. 8w+7 of all
  // four in wave order and writes them as whole 128-byte rows (eight lanes a
  // row).  Accumulator element 4 q + e of lane (n, g) is d = 8 q + 4 g + e
  // (o1: d + 32) of row n.
  constexpr int kPartRow = kD + 4;
  float* const part = reinterpret_cast<float*>(region);  // [32][68] O, [64] m, [64] l
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const float4v va = {o0[4 * q], o0[4 * q + 1], o0[4 * q + 2], o0[4 * q + 3]};
    const float4v vb = {o1[4 * q], o1[4 * q + 1], o1[4 * q + 2], o1[4 * q + 3]};
    *reinterpret_cast<float4v*>(part + n * kPartRow + 8 * q + 4 * g) = va;
    *reinterpret_cast<float4v*>(part + n * kPartRow + 32 + 8 * q + 4 * g) = vb;
  }
  part[32 * kPartRow + lane] = m;
  part[32 * kPartRow + 64 + lane] = l;
  __syncthreads();
  const int r = 8 * wave + (lane >> 3), ch = lane & 7;  // row r, columns 8 ch .. 8 ch + 7
  float M = reinterpret_cast<const float*>(lds)[32 * kPartRow + r];
#pragma unroll
  for (int w = 1; w < kWaves; ++w)
    M = fmaxf(M, reinterpret_cast<const float*>(lds + w * kRegionHalfs)[32 * kPartRow + r]);
  float lt = 0.0f;
  float4v ya = {}, yb = {};
#pragma unroll
  for (int w = 0; w < kWaves; ++w) {
    const float* pw = reinterpret_cast<const float*>(lds + w * kRegionHalfs);
    const float aw = __builtin_amdgcn_exp2f(pw[32 * kPartRow + r] - M);  // 0 for a wave with no tile
    const float4v xa = *reinterpret_cast<const float4v*>(pw + r * kPartRow + 8 * ch);
    const float4v xb = *reinterpret_cast<const float4v*>(pw + r * kPartRow + 8 * ch + 4);
    if (w == 0) {
      lt = pw[32 * kPartRow + 64 + r] * aw;
      ya = xa * aw;
      yb = xb * aw;
    } else {
      lt += pw[32 * kPartRow + 64 + r] * aw;
      ya += xa * aw;
      yb += xb * aw;
    }
  }
  const int orow = 32 * blk + r;
  if (orow < T) {
    const float inv = __builtin_amdgcn_rcpf(lt);
    const half4 ha = __builtin_convertvector(ya * inv, half4);
    const half4 hb = __builtin_convertvector(yb * inv, half4);
    const half8 o8 = {ha[0], ha[1], ha[2], ha[3], hb[0], hb[1], hb[2], hb[3]};
    *reinterpret_cast<half8*>(O + (size_t)orow * Hq * kD + (size_t)h * kD + 8 * ch) = o8;
    if (ch == 0) L[(size_t)h * T + orow] = M + __builtin_amdgcn_logf(lt);
  }
}

}  // namespace

void sattn_fwd_split_launch(const void* Q, const void* K, const void* Vt, void* O, float* L,
                            float c, int T, int Hq, int Hkv, bool vrows, hipStream_t stream) {
  const int G = Hq / Hkv;
  const int nBlocks = (T + 31) / 32;
  // pairs of query blocks (heavy n-1-j, light j) over all query heads, and
  // the grid padded so each XCD takes a whole run of pairs (see the kernel)
  const int nPairs = (nBlocks + 1) / 2 * Hq;
  const int pairsPerXcd = (nPairs + kXcds - 1) / kXcds;
  const dim3 grid((unsigned)pairsPerXcd * 2u * (unsigned)kXcds);
  const unsigned units = (unsigned)nBlocks * (unsigned)Hq;  // workgroups with work
  const half_t* q = static_cast<const half_t*>(Q);
  const half_t* k = static_cast<const half_t*>(K);
  const half_t* v = static_cast<const half_t*>(Vt);
  half_t* o = static_cast<half_t*>(O);
  // LDS staging (one workgroup per CU) when the grid fits the chip at once
  // and V comes in whole 16-byte chunks; register staging (two per CU)
  // otherwise.  The lazy reference (LDS staging only: register staging has no
  // room for its slow path) is taken exactly where the V^T entry can stage
  // through LDS, so both entries round alike at every shape.
  const bool dma = (vrows || T % 8 == 0) && units <= (unsigned)kCus;
  const bool lazy = dma && T % 8 == 0;
#define SATTN_SPLIT(VT, VR, DM, LZ)                                                                \
  hipLaunchKernelGGL((sattn_fwd_split_kernel<VT, VR, DM, LZ>), grid, dim3(64 * kWaves), 0, stream, \
                     q, k, v, o, L, c, T, Hq, G, nBlocks, nPairs, pairsPerXcd)
  if (vrows && lazy)
    SATTN_SPLIT(false, true, true, true);
  else if (vrows && dma)
    SATTN_SPLIT(false, true, true, false);
  else if (vrows)
    SATTN_SPLIT(false, true, false, false);
  else if (lazy)
    SATTN_SPLIT(true, false, true, true);
  else if (T % 8 == 0)
    SATTN_SPLIT(true, false, false, false);
  else
    SATTN_SPLIT(false, false, false, false);
#undef SATTN_SPLIT
}
