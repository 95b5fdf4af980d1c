// The causal streaming-attention forward for gfx950 (CDNA4), and its C entry.
//
// Method (StreamingAttentionSM86 page, header comment and tile body of the
// forward realization): for each 64-key tile up to the diagonal, scores are
// formed on the matrix cores, scaled to base-2 units t = S*c, folded into a
// running row maximum m, row sum l and weighted sum O by the merge rule for
// normalised weighted sums (a new reference m' scales the old l and O by
// 2^(m - m')), and the tile's P V is added with P = 2^(t - m') rounded to
// binary16.  The epilogue writes O / l (binary16, token-major) and
// m + log2 l (binary32).
//
// gfx950 design (not the page's SM86 one):
//  * The transposed problem is computed: S^T = K Q^T and O^T = V^T P^T on
//    v_mfma_f32_32x32x16_f16 with every accumulator in VGPRs.  In the 32x32
//    accumulator layout a lane holds one column (one query) and 16 rows
//    (keys), so a row's max and sum are in-lane except for one exchange with
//    the lane 32 away, and the S^T accumulator is directly the P^T operand of
//    the second product.
//  * The K rows feeding S^T are permuted (the `krow` map below) so that the
//    eight keys a lane holds for each 16-key slice of P^T are consecutive:
//    the matching V^T operand is then one 16-byte LDS read.
//  * A wave owns 32 query rows of one head.  A workgroup is eight waves (one
//    per CU): GW query heads of one GQA group times 8/GW row slots, so each
//    K/V tile staged in LDS feeds all of them.  Problems too small to give
//    every CU such a workgroup go to the split-key kernel instead.  Query
//    rows come in 32-row blocks; a slot takes block n-1-p (heavy) and then
//    block p (light), so every workgroup carries the same causal work.
//  * Each wave is software-pipelined: step j forms P V of tile j-1 and S of
//    tile j+1 on the matrix cores while its VALUs turn S of tile j into P.
//    The step is laid out by hand (scheduling barriers): each of its 16
//    matrix products reads its LDS operand four products ahead and is
//    followed by the exponentials of two scores.  Two register sets of S and
//    of binary16 P alternate between steps, so no copies carry them.  Odd
//    steps run at a higher wave priority than even ones, so the two waves
//    sharing a SIMD alternate between the workgroup's barriers.
//  * K tile t is read at steps t-1 and t, V^T tile t at step t+1.  Two K and
//    two V^T tiles are staged per barrier, every other step, into rings of 6
//    and 5 LDS buffers (101 KiB).
//    Global loads run one stage (two steps) ahead of their LDS stores through
//    registers, and every stage issues the same loads (tiles past the end
//    read as zeros through buffer-descriptor range checks, applied to the
//    loads' VGPR offsets, which carry the whole offset), so the waits on
//    them stay exact.  LDS rows are padded to 144 bytes so the 16-byte
//    operand reads of 16 lanes hit 64 distinct banks.
//  * The reference maximum is moved lazily.  P is formed against the current
//    reference; only when some lane's partial row sum leaves (0, 2^kLazy] is
//    the reference raised, by the power of two that brings the row's largest
//    P to at most 1 (exact scaling of P, l and O), or, if a P overflowed
//    binary32, from the tile's maximum score.  The merge rule holds for any
//    reference, so this changes only rounding, and P stays at most 2^kLazy.
//  * Tiles past the causal diagonal are never visited and only a query
//    block's last tile (the one crossing its diagonal) is masked.  Rows past
//    T are computed on zero queries and not stored, so T need not be a
//    multiple of 64.
//  * A block's end: each wave writes its O rows into its own LDS rows and
//    reads them back row-major, so its global stores write whole 128-byte
//    row segments; the light block's Q rows and first tiles are loaded before
//    the heavy block's O stores, whose completion the vector memory counter
//    would otherwise make those loads wait for.
//  * Workgroups are dealt to the eight XCDs round-robin; they are renumbered
//    so that each XCD receives a contiguous run ordered K/V head first,
//    keeping one K/V head's tiles in one XCD's L2.
//  * Problems with too few query blocks for eight-wave workgroups on every CU
//    go to the split-key kernel of sattn_fwd_split.hip, which walks each
//    block's key range with four waves at once.
#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>
#include <string.h>

#include <atomic>
#include <type_traits>

#include "sattn.h"
#include "sattn_internal.h"

namespace {

typedef _Float16 half_t;
typedef _Float16 half4 __attribute__((ext_vector_type(4)));
typedef _Float16 half8 __attribute__((ext_vector_type(8)));
typedef float float4v __attribute__((ext_vector_type(4)));
typedef float float8v __attribute__((ext_vector_type(8)));
typedef float float16v __attribute__((ext_vector_type(16)));
typedef int int4v __attribute__((ext_vector_type(4)));

constexpr int kD = SATTN_HEAD_DIM;  // head width
constexpr int kBN = 64;             // keys per tile
constexpr int kRowHalfs = kD + 8;                // LDS row: 64 values + 16 bytes of padding
constexpr int kTileHalfs = kBN * kRowHalfs;      // one K or V^T tile in LDS
constexpr float kLazy = 8.0f;                    // rescale threshold, base-2 units
constexpr int kBufferWord3 = 0x00020000;         // raw buffer, 32-bit data format
constexpr int kXcds = 8;                         // accelerator complex dies per MI355X
constexpr int kCus = 256;                        // compute units per MI355X
constexpr int kNW = 8;                           // waves per workgroup (one workgroup per CU)

__device__ __forceinline__ half8 to_half8(float8v x) { return __builtin_convertvector(x, half8); }

__device__ __forceinline__ float16v mfma(half8 a, half8 b, float16v c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b, c, 0, 0, 0);
}

// Maximum of 32 values as a tree of v_max3 (depth 5 instead of a 16-long
// dependent chain).
__device__ __forceinline__ float max32(const float16v& a, const float16v& b) {
  float t[8], u[4], w[2];
#pragma unroll
  for (int i = 0; i < 8; ++i) t[i] = __builtin_fmaxf(__builtin_fmaxf(a[i], a[i + 8]), b[i]);
#pragma unroll
  for (int i = 0; i < 4; ++i) u[i] = __builtin_fmaxf(__builtin_fmaxf(t[i], t[i + 4]), b[8 + i]);
#pragma unroll
  for (int i = 0; i < 2; ++i) w[i] = __builtin_fmaxf(__builtin_fmaxf(u[i], u[i + 2]), b[12 + i]);
  return __builtin_fmaxf(__builtin_fmaxf(__builtin_fmaxf(w[0], w[1]), b[14]), b[15]);
}

// Sum of 32 values as a pairwise tree (depth 5).
__device__ __forceinline__ float sum32(const float16v& a, const float16v& b) {
  float t[16];
#pragma unroll
  for (int i = 0; i < 16; ++i) t[i] = a[i] + b[i];
#pragma unroll
  for (int w = 8; w >= 1; w >>= 1)
#pragma unroll
    for (int i = 0; i < w; ++i) t[i] += t[i + w];
  return t[0];
}

// Workgroup barrier without the memory fence of __syncthreads(): callers wait
// for what the barrier publishes themselves, so global loads meant to stay in
// flight across it are not waited for.
__device__ __forceinline__ void barrier() { asm volatile("s_barrier" ::: "memory"); }

// Orders a wave's LDS writes before its reads of what other lanes of the
// same wave wrote (wavefront-scope release, wave barrier, acquire).  A wave's
// LDS operations complete in order, so this emits no wait; it keeps the
// compiler from moving the reads above the writes.
__device__ __forceinline__ void wave_lds_sync() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

// The value held by the lane whose byte address (lane index * 4) is `addr`.
__device__ __forceinline__ float xlane(float x, int addr) {
  return __builtin_bit_cast(float, __builtin_amdgcn_ds_bpermute(addr, __builtin_bit_cast(int, x)));
}

// K row loaded by A-operand row m of S^T = K Q^T, chosen so that accumulator
// element i of lane (n, g) is key 16*(i/8) + 8g + i%8 of the 32-key block.
__device__ __forceinline__ int krow(int m) {
  const int a = m >> 3, e = (m >> 2) & 1, b = m & 3;
  return 16 * (a >> 1) + 8 * e + 4 * (a & 1) + b;
}

// V given as rows ([head][T][64]) is staged like K, in unpadded 64-value rows
// whose 16-byte chunk c of row r sits at chunk c ^ vswz(r) (vswz(r) = the bits
// of (r/2) % 8 reversed), and its V^T operand is read with the LDS transpose
// read ds_read_b64_tr_b16: in each 16-lane group, lane 4a + b points at row
// a, columns 4b .. 4b+3 of a 4 x 16 block, and lane t receives column t,
// rows 0..3.  Two reads (rows k .. k+3, k+4 .. k+7) make one operand; the
// swizzle keeps the 32 lanes of a read on distinct banks.
__device__ __forceinline__ int vswz(int r) {
  const int v = (r >> 1) & 7;
  return ((v & 1) << 2) | (v & 2) | (v >> 2);
}
__device__ __forceinline__ int vchunk(int r, int c) { return r * kD + ((c ^ vswz(r)) << 3); }
__device__ __forceinline__ half4 lds_tr4(const half_t* p) {
  typedef short short4v __attribute__((ext_vector_type(4)));
  typedef __attribute__((address_space(3))) short4v lds_short4;
  const short4v v = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_short4*)(const_cast<half_t*>(p)));
  return __builtin_bit_cast(half4, v);
}
// A lane's transpose-read offset (halfs) in a V-rows tile for operand rows
// d = 32 mh .. 32 mh + 31 (d = lane % 32 + 32 mh), keys 8(lane/32) + 4 hi ..
__device__ __forceinline__ int vtr_offset(int lane, int mh, int hi) {
  const int row = 8 * (lane >> 5) + ((lane & 15) >> 2) + 4 * hi;
  const int col = 32 * mh + 16 * ((lane >> 4) & 1) + 4 * (lane & 3);
  return vchunk(row, col >> 3) + (col & 7);
}

template <int GW, bool VT_VEC, bool VROWS>
__global__ void __launch_bounds__(64 * kNW, 1)
sattn_fwd_kernel(const half_t* __restrict__ Q, const half_t* __restrict__ K,
                 const half_t* __restrict__ Vt, half_t* __restrict__ O, float* __restrict__ L,
                 float c, int T, int Hq, int Hkv, int G, int nBlocks, int nPairs, int nSlotGroups,
                 int nHeadGroups) {
  constexpr int RS = kNW / GW;             // row slots per workgroup
  // Two tiles are staged per barrier, which needs these ring depths (see the
  // stage below).
  constexpr int kKRing = 6;                // K tile t is read at steps t-1 and t
  constexpr int kVRing = 5;                // V^T tile t is read at step t+1
  constexpr float kSumCap = 256.0f;        // 2^kLazy
  // A stage's barrier runs inside the step that follows it, after this slot
  // (its LDS writes then complete under the step's first products; A/B on
  // one MI355X against a barrier before the step: +1.5 % at T=4096 and
  // T=16384, outputs bit-identical).
  constexpr int kBarrierSlot = 7;
  constexpr unsigned kOutOfRange = 0x7FFFFFF0u;  // past every plane (at most 2^31 - 128 bytes)
  __shared__ __attribute__((aligned(16))) half_t smem[(kKRing + kVRing) * kTileHalfs];
  // each wave's 32 O rows on their way to global memory (see the epilogue)
  __shared__ __attribute__((aligned(16))) half_t obuf[kNW][32 * kRowHalfs];
  half_t* const kring = smem;
  half_t* const vring = smem + kKRing * kTileHalfs;
  constexpr int kTileBytes = kTileHalfs * 2;
  // LDS operand of ring buffer `buf` at byte offset `off` from the lane's base.
  // The buffer offset goes through readfirstlane so that it stays one scalar
  // per step instead of a per-lane induction variable per read.
  auto lds8 = [&](const half_t* ring, int buf, int laneByte, int off) -> half8 {
    const int b = __builtin_amdgcn_readfirstlane(buf * kTileBytes);
    return *reinterpret_cast<const half8*>(reinterpret_cast<const char*>(ring) + laneByte + b +
                                           off);
  };

  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lane = tid & 63;
  const int n = lane & 31;
  const int g = lane >> 5;

  const int nWg = gridDim.x;
  const int xcd = blockIdx.x % kXcds, idx = blockIdx.x / kXcds;
  const int lid = xcd * (nWg / kXcds) + min(xcd, nWg % kXcds) + idx;
  const int perKv = nHeadGroups * nSlotGroups;
  const int kv = lid / perKv;
  const int hg = (lid - kv * perKv) / nSlotGroups;
  const int sg = lid - kv * perKv - hg * nSlotGroups;
  const int h = kv * G + hg * GW + (wave % GW);
  const int slot = wave / GW;

  auto block_of = [&](int task, int s) -> int {
    const int p = sg * RS + s;
    if (p >= nPairs) return -1;
    const int hi = nBlocks - 1 - p;
    return task == 0 ? hi : (p < hi ? p : -1);
  };
  auto need_of = [&](int blk) -> int { return blk < 0 ? 0 : min(T - 1, 32 * blk + 31) / kBN + 1; };

  // Global -> register staging: thread t owns 16-byte chunk t of a K tile and
  // of a V^T tile (row cr, column chunk cc).  Two register sets, by stage
  // parity, keep loads two steps ahead of their LDS stores.
  constexpr int kCpt = 8 / kNW;          // 16-byte chunks per thread per tile
  constexpr int kRowsPerPass = 8 * kNW;  // tile rows one pass of the workgroup covers
  const int cr = tid >> 3, cc = tid & 7;
  const __amdgpu_buffer_rsrc_t krsrc = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<half_t*>(K + (size_t)kv * T * kD), 0, T * kD * 2, kBufferWord3);
  // V^T of head kv, or (VROWS) V rows of head kv: the same element count
  const half_t* Vh = Vt + (size_t)kv * kD * T;
  const __amdgpu_buffer_rsrc_t vrsrc =
      __builtin_amdgcn_make_buffer_rsrc(const_cast<half_t*>(Vh), 0, kD * T * 2, kBufferWord3);
  const int kByte = (cr * kD + cc * 8) * 2;
  const unsigned vByte = ((unsigned)cr * (unsigned)T + (unsigned)cc * 8u) * 2u;
  typedef int4v Stage[kCpt];
  // The whole offset of every buffer load is in its VGPR offset, which the
  // range check covers (the scalar offset is added after the check): rows
  // past T, and whole tiles past the last, read as zeros without touching
  // memory past the head's plane.  Offsets stay below 2^31 + 2^15 for every
  // admitted shape (a plane holds at most 2^31 bytes), so they are unsigned.
  auto load_k = [&](int kt, Stage& dst) {
    const unsigned t0 = (unsigned)__builtin_amdgcn_readfirstlane(kt) * (unsigned)(kBN * kD * 2);
#pragma unroll
    for (int p = 0; p < kCpt; ++p)
      dst[p] = __builtin_amdgcn_raw_buffer_load_b128(
          krsrc, t0 + (unsigned)(kByte + p * kRowsPerPass * kD * 2), 0, 0);
  };
  // V^T chunks at or past T (T % 8 == 0: a chunk is wholly inside or
  // outside) take an offset past the buffer's range and read as zeros, so
  // every stage issues the same loads and the waits stay exact.
  auto load_v = [&](int kt, Stage& dst) {
    const int key0 = kt * kBN;
#pragma unroll
    for (int p = 0; p < kCpt; ++p) {
      const unsigned rb = (unsigned)vByte + (unsigned)(p * kRowsPerPass) * (unsigned)T * 2u;
      if (VROWS) {  // rows past T read as zeros, like K's
        const unsigned t0 = (unsigned)__builtin_amdgcn_readfirstlane(kt) * (unsigned)(kBN * kD * 2);
        dst[p] = __builtin_amdgcn_raw_buffer_load_b128(
            vrsrc, t0 + (unsigned)(kByte + p * kRowsPerPass * kD * 2), 0, 0);
      } else if (VT_VEC) {
        const unsigned off = key0 + cc * 8 < T ? rb + (unsigned)key0 * 2u : (unsigned)kOutOfRange;
        dst[p] = __builtin_amdgcn_raw_buffer_load_b128(vrsrc, off, 0, 0);
      } else if (key0 + kBN <= T) {
        dst[p] = __builtin_amdgcn_raw_buffer_load_b128(vrsrc, rb + (unsigned)key0 * 2u, 0, 0);
      } else {
        const half_t* vsrc = Vh + (size_t)(cr + p * kRowsPerPass) * T + key0 + cc * 8;
        half8 v;
#pragma unroll
        for (int e = 0; e < 8; ++e) v[e] = (key0 + cc * 8 + e < T) ? vsrc[e] : (half_t)0;
        dst[p] = __builtin_bit_cast(int4v, v);
      }
    }
  };
  const int stOff = cr * kRowHalfs + cc * 8;
  auto store_k = [&](int buf, const Stage& src) {
    const int b = __builtin_amdgcn_readfirstlane(buf * kTileBytes);
#pragma unroll
    for (int p = 0; p < kCpt; ++p)
      *reinterpret_cast<int4v*>(reinterpret_cast<char*>(kring) + b +
                                (stOff + p * kRowsPerPass * kRowHalfs) * 2) = src[p];
  };
  auto store_v = [&](int buf, const Stage& src) {
    const int b = __builtin_amdgcn_readfirstlane(buf * kTileBytes);
#pragma unroll
    for (int p = 0; p < kCpt; ++p) {
      const int off = VROWS ? vchunk(cr + p * kRowsPerPass, cc) : stOff + p * kRowsPerPass * kRowHalfs;
      *reinterpret_cast<int4v*>(reinterpret_cast<char*>(vring) + b + off * 2) = src[p];
    }
  };

  const int swapAddr = (lane ^ 32) << 2;
  const int kOff = krow(n) * kRowHalfs + 8 * g;
  const int vOff = n * kRowHalfs + 8 * g;
  int vtrOff[2][2];  // VROWS: transpose-read offsets, d rows 32 mh .., keys 4 hi ..
#pragma unroll
  for (int mh = 0; mh < 2; ++mh)
#pragma unroll
    for (int hi = 0; hi < 2; ++hi) vtrOff[mh][hi] = VROWS ? vtr_offset(lane, mh, hi) : 0;
  // V^T operand of P V from ring buffer `buf`: keys 16 ks4 + 8g .. +7 of the
  // tile, d rows 32 mh + n; from a V^T tile (one 16-byte read) or, with
  // VROWS, from a V-rows tile (two transpose reads)
  auto vt_operand = [&](int buf, int ks4, int mh) -> half8 {
    if constexpr (VROWS) {
      const half_t* base = reinterpret_cast<const half_t*>(
          reinterpret_cast<const char*>(vring) + __builtin_amdgcn_readfirstlane(buf * kTileBytes)) +
          16 * ks4 * kD;
      const half4 lo = lds_tr4(base + vtrOff[mh][0]);
      const half4 hi = lds_tr4(base + vtrOff[mh][1]);
      return half8{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
    } else {
      return lds8(vring, buf, vOff * 2, (32 * mh * kRowHalfs + 16 * ks4) * 2);
    }
  };

  auto tiles_of = [&](int task) -> int {
    int nkt = 0;
#pragma unroll
    for (int s = 0; s < RS; ++s) nkt = max(nkt, need_of(block_of(task, s)));
    return nkt;
  };
  // A task's Q rows and first K and V^T tiles, loaded into registers before
  // the task starts: for the second task, ahead of the first task's O
  // stores, whose completion the wait for these loads would otherwise
  // include (the vector memory counter retires loads and stores in order).
  half8 qn[4];
  Stage pk[2], setK[2], setV[2];
  auto prefetch = [&](int task) {
    const int blk = block_of(task, slot);
    const int need = need_of(blk);
    const int row = 32 * max(blk, 0) + n;
    const half_t* qrow = Q + ((size_t)h * T + row) * kD + 8 * g;
#pragma unroll
    for (int kk = 0; kk < 4; ++kk)
      qn[kk] = (need > 0 && row < T) ? *reinterpret_cast<const half8*>(qrow + 16 * kk) : half8{};
    load_k(0, pk[0]);
    load_k(1, pk[1]);
    load_k(2, setK[0]);
    load_v(0, setV[0]);
    load_k(3, setK[1]);
    load_v(1, setV[1]);
  };
  prefetch(0);

#pragma nounroll
  for (int task = 0; task < 2; ++task) {
    const int nkt = tiles_of(task);
    if (nkt == 0) break;
    const int blk = block_of(task, slot);
    const int need = need_of(blk);
    const int row = 32 * max(blk, 0) + n;

    half8 qf[4];
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) qf[kk] = qn[kk];
    float m = -INFINITY, l = 0.0f;
    float16v o0 = {}, o1 = {};
    float16v sa0, sa1, sb0, sb1;
    half8 pa[4], pb[4];

    auto scores = [&](int buf, float16v& r0, float16v& r1) {
#pragma unroll
      for (int kk = 0; kk < 4; ++kk) {
        const half8 a0 = lds8(kring, buf, kOff * 2, 32 * kk);
        const half8 a1 = lds8(kring, buf, kOff * 2, (32 * kRowHalfs + 16 * kk) * 2);
        r0 = mfma(a0, qf[kk], kk == 0 ? float16v{} : r0);
        r1 = mfma(a1, qf[kk], kk == 0 ? float16v{} : r1);
      }
    };
    auto pv = [&](int buf, const half8 (&p)[4]) {
#pragma unroll
      for (int ks4 = 0; ks4 < 4; ++ks4) {
        const half8 v0 = vt_operand(buf, ks4, 0);
        const half8 v1 = vt_operand(buf, ks4, 1);
        o0 = mfma(v0, p[ks4], o0);
        o1 = mfma(v1, p[ks4], o1);
      }
    };
    auto mask = [&](int j, float16v& s0, float16v& s1) {
      const int lim = row - j * kBN - 8 * g;
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const int k = 16 * (i >> 3) + (i & 7);
        if (k > lim) s0[i] = -INFINITY;
        if (k + 32 > lim) s1[i] = -INFINITY;
      }
    };
    auto exp_tile = [&](float16v& s0, float16v& s1) -> float {
      const float neg_m = -m;
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        s0[i] = __builtin_amdgcn_exp2f(__builtin_fmaf(s0[i], c, neg_m));
        s1[i] = __builtin_amdgcn_exp2f(__builtin_fmaf(s1[i], c, neg_m));
      }
      return sum32(s0, s1);
    };
    auto round_p = [&](const float16v& s0, const float16v& s1, half8 (&p)[4]) {
      p[0] = to_half8(__builtin_shufflevector(s0, s0, 0, 1, 2, 3, 4, 5, 6, 7));
      p[1] = to_half8(__builtin_shufflevector(s0, s0, 8, 9, 10, 11, 12, 13, 14, 15));
      p[2] = to_half8(__builtin_shufflevector(s1, s1, 0, 1, 2, 3, 4, 5, 6, 7));
      p[3] = to_half8(__builtin_shufflevector(s1, s1, 8, 9, 10, 11, 12, 13, 14, 15));
    };
    auto exact_reference = [&](const float16v& s0, const float16v& s1) {
      const float x = max32(s0, s1);
      const float mx = __builtin_fmaxf(x, xlane(x, swapAddr)) * c;
      const float m_new = __builtin_fmaxf(m, mx);
      const float alpha = __builtin_amdgcn_exp2f(m - m_new);  // 0 when m = -inf
      m = m_new;
      l *= alpha;
      o0 *= alpha;
      o1 *= alpha;
    };

    // Step j >= 1: P V of tile j-1 (pin), S of tile j+1 into x (SN), P of
    // tile j from its scores in s into pout (masked on the query block's
    // last tile).  The fast path is laid out by hand: the LDS operand of
    // each matrix product is read four products ahead, and every product is
    // followed by the softmax of two score elements; scheduling barriers
    // keep that order.
    // `bar`: this step carries the barrier of the stage issued just before it
    // (see the stage below), after its eighth slot.
    auto step = [&](auto SNF, auto MASKF, int j, float16v& s0, float16v& s1, float16v& x0,
                    float16v& x1, const half8 (&pin)[4], half8 (&pout)[4], bool bar) {
      constexpr bool kSn = decltype(SNF)::value, kMask = decltype(MASKF)::value;
      constexpr int kM = kSn ? 16 : 8;  // matrix products this step
      const int vbuf = (j + kVRing - 1) % kVRing, kbuf = (j + 1) % kKRing;
      auto rd = [&](int i) -> half8 {
        if (i < 8)  // V^T operand of P V: slice ks4 = i/2, d rows 32*(i%2)
          return vt_operand(vbuf, i >> 1, i & 1);
        const int kk = (i - 8) >> 1, sb = i & 1;  // K operand of S: k-step kk, key rows 32*sb
        return lds8(kring, kbuf, kOff * 2, (32 * sb * kRowHalfs + 16 * kk) * 2);
      };
      // Odd steps run at the higher wave priority.  Of the two waves on a
      // SIMD, the one in its odd step (between the workgroup's barriers)
      // then goes first, so the pair alternates rather than the older wave
      // running ahead and waiting at the barrier (A/B on one MI355X, outputs
      // bit-identical: +1 to +2.7 % at T=4096, +1.2 % at T=16384).
      if (j & 1) __builtin_amdgcn_s_setprio(1);
      else __builtin_amdgcn_s_setprio(0);
      if constexpr (kMask) mask(j, s0, s1);
      const float neg_m = -m;
      half8 r[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) r[i] = rd(i);
      float acc[4];
      // Softmax software-pipelined across the 16 slots: slot i exponentiates
      // the two arguments formed in slot i-1, forms those of slot i+1 and
      // sums the two P of slot i-1, so no instruction waits on the one
      // issued just before it.
      auto el = [&](int e) -> float { return e < 16 ? s0[e] : s1[e - 16]; };
      auto set = [&](int e, float v) {
        if (e < 16) s0[e] = v;
        else s1[e - 16] = v;
      };
      float ta = __builtin_fmaf(el(0), c, neg_m), tb = __builtin_fmaf(el(1), c, neg_m);
      auto finish = [&](int i) {  // sum and pack the P of slot i
        const float t = el(2 * i) + el(2 * i + 1);
        acc[i & 3] = i < 4 ? t : acc[i & 3] + t;
        if ((i & 3) == 3) {
          const float16v& sv = i < 8 ? s0 : s1;  // binary16 P of keys 8(i/4 % 2) + 0..7
          const float8v v8 = (i & 4) ? __builtin_shufflevector(sv, sv, 8, 9, 10, 11, 12, 13, 14, 15)
                                     : __builtin_shufflevector(sv, sv, 0, 1, 2, 3, 4, 5, 6, 7);
          pout[i >> 2] = to_half8(v8);
        }
      };
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        if (i < kM) {
          const half8 a = r[i & 3];
          if (i < 8) {
            if (i & 1) o1 = mfma(a, pin[i >> 1], o1);
            else o0 = mfma(a, pin[i >> 1], o0);
          } else {
            const int kk = (i - 8) >> 1;
            if (i & 1) x1 = mfma(a, qf[kk], kk == 0 ? float16v{} : x1);
            else x0 = mfma(a, qf[kk], kk == 0 ? float16v{} : x0);
          }
          if (i + 4 < kM) r[i & 3] = rd(i + 4);
        }
        set(2 * i, __builtin_amdgcn_exp2f(ta));
        set(2 * i + 1, __builtin_amdgcn_exp2f(tb));
        if (i < 15) {
          ta = __builtin_fmaf(el(2 * i + 2), c, neg_m);
          tb = __builtin_fmaf(el(2 * i + 3), c, neg_m);
        }
        if (i > 0) finish(i - 1);
        __builtin_amdgcn_sched_barrier(0);
        if (i == kBarrierSlot && bar) {
          // The stage's LDS writes precede every operand read of this step,
          // and those up to slot i have been waited for; wave LDS operations
          // complete in order, so only the four youngest reads can be
          // outstanding.
          __builtin_amdgcn_s_waitcnt(0xC07F | (4 << 8));
          barrier();
          __builtin_amdgcn_sched_barrier(0);
        }
      }
      finish(15);
      float lsum = (acc[0] + acc[1]) + (acc[2] + acc[3]);
      const bool over = __builtin_amdgcn_ballot_w64(!(lsum <= kSumCap)) != 0;
      // Pins the binary16 P in this block: the fp32 P dies here on the fast
      // path, and only pout merges with the slow path.
      asm volatile("" ::"v"(pout[0]), "v"(pout[1]), "v"(pout[2]), "v"(pout[3]));
      if (over) {
        asm volatile("");  // keeps the slow path a branch, never speculated
        // Some row's partial sum left (0, 2^kLazy].  Move each row's
        // reference up by the power of two that brings its largest P to at
        // most 1; exact scaling of P, l and O.  If a P overflowed binary32,
        // S is formed again from K (still in the ring) and the reference is
        // taken from the tile maximum.
        const float x = max32(s0, s1);
        const float pmax = __builtin_fmaxf(x, xlane(x, swapAddr));
        if (__builtin_amdgcn_ballot_w64(!(pmax < INFINITY)) == 0) {
          const int e = pmax > 1.0f ? __builtin_amdgcn_frexp_expf(pmax) : 0;
          const float alpha = __builtin_ldexpf(1.0f, -e);
          m += (float)e;
          l *= alpha;
          o0 *= alpha;
          o1 *= alpha;
          s0 *= alpha;
          s1 *= alpha;
          lsum = sum32(s0, s1);
        } else {
          scores(j % kKRing, s0, s1);
          if constexpr (kMask) mask(j, s0, s1);
          exact_reference(s0, s1);
          lsum = exp_tile(s0, s1);
        }
        round_p(s0, s1, pout);
      }
      l += lsum;
    };

    // Ring schedule: K tile t is read at steps t-1 (S of t) and t (overflow
    // fallback), V^T tile t at step t+1 (P V of t); see the stage itself.
    store_k(0, pk[0]);
    store_k(1, pk[1]);
    __builtin_amdgcn_s_waitcnt(0xC07F);
    barrier();
    // Loads past the last tile read zeros and stores of them land in ring
    // buffers that are free by the same argument as real tiles, so a stage
    // has no branches.
    auto stage = [&](auto PARF, int j, bool wait = true) {
      constexpr int P = decltype(PARF)::value;
      // Even j only: K of tiles j+2, j+3 and V^T of tiles j, j+1 (loaded at
      // stage j-2) go into buffers whose tiles were last read at step j-3,
      // before the previous barrier (j-2); other waves may still be in steps
      // j-2, j-1, which read K of tiles j-2 .. j and V^T of tiles j-3, j-2 —
      // other buffers.  Then K of tiles j+4, j+5 and V^T of tiles j+2, j+3
      // are loaded into the same registers.  The first reads of the new
      // tiles are in step j+1 (S of tile j+2, P V of tile j), so the barrier
      // that publishes them may sit inside step j (`wait` false: the step
      // carries it).
      if constexpr (P == 0) {
        store_k((j + 2) % kKRing, setK[0]);
        store_k((j + 3) % kKRing, setK[1]);
        store_v(j % kVRing, setV[0]);
        store_v((j + 1) % kVRing, setV[1]);
        load_k(j + 4, setK[0]);
        load_k(j + 5, setK[1]);
        load_v(j + 2, setV[0]);
        load_v(j + 3, setV[1]);
        if (wait) {
          __builtin_amdgcn_s_waitcnt(0xC07F);
          barrier();
        }
      }
    };
    using T1 = std::integral_constant<bool, true>;
    using F0 = std::integral_constant<bool, false>;
    using P0 = std::integral_constant<int, 0>;
    using P1 = std::integral_constant<int, 1>;
    auto stage_any = [&](int j) {
      if (j & 1) stage(P1{}, j);
      else stage(P0{}, j);
    };
    // step 0: S of tiles 0 and 1, P of tile 0 from its exact maximum
    if (need > 0) scores(0, sa0, sa1);
    stage(P0{}, 0);
    if (need > 1) {
      scores(1, sb0, sb1);
      exact_reference(sa0, sa1);
      l += exp_tile(sa0, sa1);
      round_p(sa0, sa1, pa);
    } else if (need == 1) {
      mask(0, sa0, sa1);
      exact_reference(sa0, sa1);
      l += exp_tile(sa0, sa1);
      round_p(sa0, sa1, pa);
    }
    // Every wave runs stage(j) for j = 1 .. nkt-1 in order (the workgroup's
    // barriers; stage nkt would only stage tiles past every wave's last, so
    // all waves skip it); its own steps end at its own last tile: steady
    // steps 1 .. need-2 (two per trip, S and P sets alternating), the masked
    // step need-1, then P V of tile need-1 and the epilogue at step need.
    int j = 1;
    for (; j + 2 < need; j += 2) {
      stage(P1{}, j);
      step(T1{}, F0{}, j, sb0, sb1, sa0, sa1, pa, pb, false);
      stage(P0{}, j + 1, false);
      step(T1{}, F0{}, j + 1, sa0, sa1, sb0, sb1, pb, pa, true);
    }
    if (j + 1 < need) {
      stage(P1{}, j);
      step(T1{}, F0{}, j, sb0, sb1, sa0, sa1, pa, pb, false);
      ++j;
      sb0 = sa0;
      sb1 = sa1;
#pragma unroll
      for (int i = 0; i < 4; ++i) pa[i] = pb[i];
    }
    if (j + 1 == need) {
      if (j & 1) stage(P1{}, j, false);
      else stage(P0{}, j, false);
      step(F0{}, T1{}, j, sb0, sb1, sa0, sa1, pa, pb, (j & 1) == 0);
      ++j;
#pragma unroll
      for (int i = 0; i < 4; ++i) pa[i] = pb[i];
    }
    float inv = 0.0f, lse = 0.0f;
    if (need > 0) {
      if (j < nkt) stage_any(j);
      pv((j + kVRing - 1) % kVRing, pa);
      const float lt = l + xlane(l, swapAddr);
      inv = __builtin_amdgcn_rcpf(lt);
      lse = m + __builtin_amdgcn_logf(lt);
      ++j;
    }
    for (; j < nkt; ++j) stage_any(j);
    if (task == 0 && tiles_of(1) > 0) prefetch(1);
    if (need > 0) {
      // O goes through the wave's own LDS rows so that each global store
      // writes whole 128-byte row segments (eight lanes a row) rather than
      // 8 bytes in each of 32 rows.  Accumulator element 4 q4 + e of lane
      // (n, g) is d = 8 q4 + 4 g + e (o1: d + 32) of row n.  The wave reads
      // back only what its own lanes wrote.
      half_t* const ob = obuf[wave];
#pragma unroll
      for (int q4 = 0; q4 < 4; ++q4) {
        const float4v va = {o0[4 * q4], o0[4 * q4 + 1], o0[4 * q4 + 2], o0[4 * q4 + 3]};
        const float4v vb = {o1[4 * q4], o1[4 * q4 + 1], o1[4 * q4 + 2], o1[4 * q4 + 3]};
        half_t* const orow = ob + n * kRowHalfs + 8 * q4 + 4 * g;
        *reinterpret_cast<half4*>(orow) = __builtin_convertvector(va * inv, half4);
        *reinterpret_cast<half4*>(orow + 32) = __builtin_convertvector(vb * inv, half4);
      }
      wave_lds_sync();
      const int row0 = 32 * blk, rr = lane >> 3, ch = lane & 7;
#pragma unroll
      for (int p = 0; p < 4; ++p) {  // rows 8p + lane/8, 16-byte chunk lane%8
        const int r = 8 * p + rr;
        const int4v v = *reinterpret_cast<const int4v*>(ob + r * kRowHalfs + 8 * ch);
        if (row0 + r < T)
          *reinterpret_cast<int4v*>(O + (size_t)(row0 + r) * Hq * kD + (size_t)h * kD + 8 * ch) = v;
      }
      if (row < T && g == 0) L[(size_t)h * T + row] = lse;
    }
    barrier();
  }
}

// Per-device cache of "is gfx950": 0 unknown, 1 yes, 2 no.
constexpr int kMaxDevices = 64;
std::atomic<int> g_arch_ok[kMaxDevices];

int check_device() {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0) return SATTN_ERR_DEVICE;
  if (dev < kMaxDevices) {
    const int cached = g_arch_ok[dev].load(std::memory_order_relaxed);
    if (cached != 0) return cached == 1 ? SATTN_OK : SATTN_ERR_DEVICE;
  }
  hipDeviceProp_t prop;
  if (hipGetDeviceProperties(&prop, dev) != hipSuccess) return SATTN_ERR_DEVICE;
  const bool ok = strncmp(prop.gcnArchName, "gfx950", 6) == 0;
  if (dev < kMaxDevices) g_arch_ok[dev].store(ok ? 1 : 2, std::memory_order_relaxed);
  return ok ? SATTN_OK : SATTN_ERR_DEVICE;
}

// Eight-wave workgroups, one per CU; problems too small to give every CU one
// go to the split-key kernel instead (see forward()).
template <int GW, bool VT_VEC, bool VROWS>
void launch(const half_t* Q, const half_t* K, const half_t* Vt, half_t* O, float* L, float c,
            int T, int Hq, int Hkv, hipStream_t stream) {
  constexpr int RS = kNW / GW;
  const int G = Hq / Hkv;
  const int nBlocks = (T + 31) / 32;
  const int nPairs = (nBlocks + 1) / 2;
  const int nSlotGroups = (nPairs + RS - 1) / RS;
  const int nHeadGroups = G / GW;
  const unsigned grid = (unsigned)nSlotGroups * (unsigned)Hkv * (unsigned)nHeadGroups;
  hipLaunchKernelGGL((sattn_fwd_kernel<GW, VT_VEC, VROWS>), dim3(grid), dim3(64 * kNW), 0,
                     stream, Q, K, Vt, O, L, c, T, Hq, Hkv, G, nBlocks, nPairs, nSlotGroups,
                     nHeadGroups);
}

// V^T chunks of 8 keys are whole 16-byte loads only when T % 8 == 0; V rows
// are always whole 128-byte rows.
template <int GW, bool VROWS>
void launch_gw(const half_t* Q, const half_t* K, const half_t* V, half_t* O, float* L, float c,
               int T, int Hq, int Hkv, hipStream_t stream) {
  if (VROWS)
    launch<GW, false, true>(Q, K, V, O, L, c, T, Hq, Hkv, stream);
  else if (T % 8 == 0)
    launch<GW, true, false>(Q, K, V, O, L, c, T, Hq, Hkv, stream);
  else
    launch<GW, false, false>(Q, K, V, O, L, c, T, Hq, Hkv, stream);
}

template <bool VROWS>
int forward(const void* Q, const void* K, const void* V, void* O, float* L, float c, int T,
            int Hq, int Hkv, void* stream) {
  const int st = sattn_fwd_check(Q, K, V, O, L, c, T, Hq, Hkv);
  if (st != SATTN_OK) return st;
  const int dst = check_device();
  if (dst != SATTN_OK) return dst;
  const half_t* q = static_cast<const half_t*>(Q);
  const half_t* k = static_cast<const half_t*>(K);
  const half_t* v = static_cast<const half_t*>(V);
  half_t* o = static_cast<half_t*>(O);
  hipStream_t s = static_cast<hipStream_t>(stream);
  const int G = Hq / Hkv;
  const int GW = G % 4 == 0 ? 4 : G % 2 == 0 ? 2 : 1;
  const int nPairs = ((T + 31) / 32 + 1) / 2;
  const long long grid8 = (long long)((nPairs + 8 / GW - 1) / (8 / GW)) * Hkv * (G / GW);
  if (grid8 < kCus) {
    // too few query blocks to fill the chip with eight-wave workgroups: split
    // each block's key range over the four waves of a workgroup instead
    sattn_fwd_split_launch(Q, K, V, O, L, c, T, Hq, Hkv, VROWS, s);
    return hipGetLastError() == hipSuccess ? SATTN_OK : SATTN_ERR_LAUNCH;
  }
  if (G % 4 == 0)
    launch_gw<4, VROWS>(q, k, v, o, L, c, T, Hq, Hkv, s);
  else if (G % 2 == 0)
    launch_gw<2, VROWS>(q, k, v, o, L, c, T, Hq, Hkv, s);
  else
    launch_gw<1, VROWS>(q, k, v, o, L, c, T, Hq, Hkv, s);
  return hipGetLastError() == hipSuccess ? SATTN_OK : SATTN_ERR_LAUNCH;
}

}  // namespace

extern "C" int sattn_fwd(const void* Q, const void* K, const void* Vt, void* O, float* L,
                         float c, int T, int Hq, int Hkv, void* stream) {
  return forward<false>(Q, K, Vt, O, L, c, T, Hq, Hkv, stream);
}

extern "C" int sattn_fwd_vrows(const void* Q, const void* K, const void* V, void* O, float* L,
                               float c, int T, int Hq, int Hkv, void* stream) {
  return forward<true>(Q, K, V, O, L, c, T, Hq, Hkv, stream);
}
