// The backward of causal streaming attention for gfx950 (CDNA4): the query
// launch (row term D and dQ), the key launch (dK and dV^T, one plane per
// query head) and the grouped gradient reduction, with their C entries.
//
// Method (StreamingAttentionSM86 page: the comment opening the backward pass
// and those of its query launch, key launch and grouped reduction): P is
// recomputed from the forward's base-2 log-sum-exp, P = 2^(S c - L); with
// dP = dO V^T and D = rowsum(dO * O), dS = P (dP - D); then dQ = s dS K,
// dK = s dS^T Q and dV = P^T dO.  The query launch walks the key tiles up to
// its rows' diagonal keeping dQ; the key launch walks the query tiles from
// its keys' diagonal to the end keeping dK and dV.  S and dP are formed in
// both launches, so neither needs the other's partial sums: there are no
// atomics, and every sum is taken in a fixed order.  P and dS are rounded to
// binary16 as operands of the products that follow (P for dV, dS for dQ and
// dK); all accumulation is binary32.
//
// gfx950 design (not the page's SM86 one):
//  * Products run on v_mfma_f32_32x32x16_f16.  Its two operands take, per
//    lane, eight consecutive elements along the contraction, and its
//    accumulator gives a lane one column and 16 rows.  Each launch picks the
//    orientation whose accumulator feeds the next product directly: the
//    query launch forms S^T and dP^T (a lane holds one query, so L and D are
//    per-lane constants) and the key launch S and dP (a lane holds one key).
//    The row order of the natural operand is permuted (krow) so that the
//    accumulator's 16 rows per lane are the 2 x 8 consecutive indices the
//    following product contracts over.
//  * Operands that the products need along the other axis of a tile staged
//    in LDS (K^T and V rows from the V^T tile in the query launch; Q^T and
//    dO^T in the key launch) are read with ds_read_b64_tr_b16, the LDS
//    transpose read: a 16-lane group whose lanes point at four rows of a
//    16-column block receives that block transposed, four consecutive rows
//    per lane.  Two such reads make one operand, so the backward consumes the
//    forward's own layouts (Q, K, V^T, token-major O) and no transposed copy
//    of anything is written to memory.
//  * A wave owns 32 queries (query launch) or 32 keys (key launch); a
//    workgroup is eight (or, on small grids, four) waves on consecutive rows
//    and stages each 64-row tile once for all of them, loaded two tiles
//    ahead.  On large grids a workgroup takes a heavy block and then its
//    light partner (blocks b and n-1-b), so every workgroup carries the same
//    causal work; each XCD receives a contiguous run of workgroups ordered
//    K/V head first (that head's tiles stay in its L2).
//  * With GQA the key launch writes one dK and one dV^T plane per query head
//    into a caller-provided workspace and a reduction sums the G planes of
//    each K/V head in head order; with Hq == Hkv it writes dK and dV^T
//    directly.
#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>
#include <string.h>

#include <atomic>

#include "sattn.h"
#include "sattn_check.h"
#include "sattn_lds.h"

namespace {

typedef _Float16 half_t;
typedef _Float16 half4 __attribute__((ext_vector_type(4)));
typedef _Float16 half8 __attribute__((ext_vector_type(8)));
typedef float float4v __attribute__((ext_vector_type(4)));
typedef float float16v __attribute__((ext_vector_type(16)));
typedef int int4v __attribute__((ext_vector_type(4)));

constexpr int kD = SATTN_HEAD_DIM;              // head width
constexpr int kTile = 64;                       // rows of a staged K, V^T, Q or dO tile
constexpr int kRowHalfs = sattn_lds::kRowHalfs; // LDS row: 64 values, 16-byte chunks swizzled
constexpr int kTileHalfs = kTile * kRowHalfs;
constexpr int kBufferWord3 = 0x00020000;        // raw buffer, 32-bit data format
constexpr int kOutOfRange = 0x7FFFFFF0;         // a buffer offset past every range
constexpr int kCus = 256;                       // compute units per MI355X
constexpr int kXcds = 8;                        // accelerator complex dies per MI355X

// Workgroups are dealt to the eight XCDs round-robin by index.  This returns
// the workgroup's place in an order where each XCD receives one contiguous
// run, so a run that covers one K/V head keeps that head's tiles in one L2.
__device__ __forceinline__ int xcd_order() {
  const int n = gridDim.x, b = blockIdx.x;
  const int xcd = b % kXcds, idx = b / kXcds;
  return xcd * (n / kXcds) + min(xcd, n % kXcds) + idx;
}

// The split launches' order: 32-row blocks are paired, heavy with light (the
// pair's causal work is about constant), and pairs numbered K/V head first,
// then the pair index j, then the group's query heads.  XCD x takes the
// contiguous run of pairs x * pairsPerXcd ..: its first pairsPerXcd
// workgroups take the pairs' heavy blocks (heaviest first) and the next
// pairsPerXcd their light blocks, so the XCDs carry equal work and two
// workgroups sharing a CU form one pair.  Returns false for the grid's
// padding and for the missing partner of an odd middle block; otherwise sets
// the K/V head, the query head and j, with `light` telling which member.
__device__ __forceinline__ bool split_unit(int nBlocks, int G, int nPairs, int pairsPerXcd, int& kv,
                                           int& h, int& j, bool& light) {
  const int xcd = blockIdx.x % kXcds, pos = blockIdx.x / kXcds;
  light = pos >= pairsPerXcd;
  const int pair = xcd * pairsPerXcd + (light ? pos - pairsPerXcd : pos);
  if (pair >= nPairs) return false;
  const int perKv = ((nBlocks + 1) / 2) * G;
  kv = pair / perKv;
  j = (pair - kv * perKv) / G;
  h = kv * G + (pair - kv * perKv) % G;
  return !(light && j >= nBlocks - 1 - j);
}

__device__ __forceinline__ float16v mfma(half8 a, half8 b, float16v c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b, c, 0, 0, 0);
}

// The value held by the lane whose byte address (lane index * 4) is `addr`.
__device__ __forceinline__ float xlane(float x, int addr) {
  return __builtin_bit_cast(float, __builtin_amdgcn_ds_bpermute(addr, __builtin_bit_cast(int, x)));
}

// Row of the natural operand loaded by operand row m, chosen so that
// accumulator element i of lane (n, g) is index 16*(i/8) + 8g + i%8 of the
// 32-row block: bits 2 and 3 of m swapped.
__device__ __forceinline__ int krow(int m) {
  const int a = m >> 3, e = (m >> 2) & 1, b = m & 3;
  return 16 * (a >> 1) + 8 * e + 4 * (a & 1) + b;
}

__device__ __forceinline__ half8 ld8(const half_t* p) { return *reinterpret_cast<const half8*>(p); }

// Workgroup barrier without __syncthreads()'s wait for every outstanding
// load: callers wait for their LDS stores (kLdsDone) and let the global loads
// of later tiles stay in flight across it.
__device__ __forceinline__ void barrier() { asm volatile("s_barrier" ::: "memory"); }
constexpr int kLdsDone = 0xC07F;  // s_waitcnt lgkmcnt(0), other counters unconstrained

using sattn_lds::chunk_offset;
using sattn_lds::tr8;
using sattn_lds::tr_offset;

// binary16 operand of 16 consecutive indices from accumulator elements
// 8h .. 8h+7 (round to nearest even).
__device__ __forceinline__ half8 pack8(const float16v& x, int h) {
  half8 r;
#pragma unroll
  for (int e = 0; e < 8; ++e) r[e] = (half_t)x[8 * h + e];
  return r;
}

// -------------------------------------------------------------------------
// Query launch: D and dQ.  Workgroup = NW waves x 32 query rows of head h.
// -------------------------------------------------------------------------
template <int NW, bool VT_VEC, bool PAIRED>
__global__ void __launch_bounds__(64 * NW, 8 / NW)
sattn_bwdq_kernel(const half_t* __restrict__ Q, const half_t* __restrict__ K,
                  const half_t* __restrict__ Vt, const half_t* __restrict__ O,
                  const half_t* __restrict__ dO, const float* __restrict__ L,
                  float* __restrict__ dQ, float* __restrict__ D, float c, float s, int T, int Hq,
                  int G, int nBlocks, int nPairs) {
  __shared__ __attribute__((aligned(16))) half_t smem[4 * kTileHalfs];
  half_t* const kbuf = smem;                   // K tiles [2][64 keys][64], chunks swizzled
  half_t* const vbuf = smem + 2 * kTileHalfs;  // V^T tiles [2][64 d][64], chunks swizzled

  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lane = tid & 63;
  const int n = lane & 31;
  const int g = lane >> 5;

  // K/V head first, then query blocks heaviest first (paired: heavy block
  // nBlocks-1-p, then light block p, so every workgroup carries the same
  // causal work), then the group's heads
  const int lid = xcd_order();
  const int kv = lid / (nPairs * G);
  const int rem = lid - kv * nPairs * G;
  const int pair = rem / G;
  const int h = kv * G + rem % G;
  auto run = [&](int blk) {
    const int row0 = blk * 32 * NW;
    const int waveRow0 = row0 + 32 * wave;
    const int row = waveRow0 + n;
    const bool live = row < T;
    const int nkt = min(T - 1, row0 + 32 * NW - 1) / kTile + 1;  // key tiles of the workgroup
    const int waveLast = min(T - 1, waveRow0 + 31);               // the wave's last row

    // Q and dO rows as B operands (lane: row n, columns 16kk + 8g .. +7), and D.
    half8 qf[4], dof[4];
    float dpart = 0.0f;
    {
      const half_t* qrow = Q + ((size_t)h * T + row) * kD + 8 * g;
      const size_t tok = (size_t)row * Hq * kD + (size_t)h * kD + 8 * g;
  #pragma unroll
      for (int kk = 0; kk < 4; ++kk) {
        const half8 z = {};
        qf[kk] = live ? ld8(qrow + 16 * kk) : z;
        dof[kk] = live ? *reinterpret_cast<const half8*>(dO + tok + 16 * kk) : z;
        const half8 of = live ? *reinterpret_cast<const half8*>(O + tok + 16 * kk) : z;
  #pragma unroll
        for (int e = 0; e < 8; ++e) dpart = fmaf((float)dof[kk][e], (float)of[e], dpart);
      }
    }
    const float Drow = dpart + xlane(dpart, (lane ^ 32) << 2);
    const float negL = live ? -L[(size_t)h * T + row] : 0.0f;
    float16v negD;
  #pragma unroll
    for (int i = 0; i < 16; ++i) negD[i] = -Drow;
    if (live && g == 0) D[(size_t)h * T + row] = Drow;

    // Staging: thread t owns 16-byte chunks t, t + 64 NW, .. of a K tile (row
    // c/8, column chunk c%8) and of a V^T tile.
    constexpr int kCpt = 512 / (64 * NW), kRowStep = 8 * NW;  // chunks per thread, rows between them
    const int cr = tid >> 3, cc = tid & 7;
    const __amdgpu_buffer_rsrc_t krsrc = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<half_t*>(K + (size_t)kv * T * kD), 0, T * kD * 2, kBufferWord3);
    const half_t* Vh = Vt + (size_t)kv * kD * T;
    const __amdgpu_buffer_rsrc_t vrsrc =
        __builtin_amdgcn_make_buffer_rsrc(const_cast<half_t*>(Vh), 0, kD * T * 2, kBufferWord3);
    // Two register sets by tile parity: tile kt + 2 is loaded at step kt and
    // stored at step kt + 1, so its loads have a whole step to arrive.  Tiles
    // past the end read as zeros (range checks), so every step issues the same
    // loads and stores and the compiler's load waits stay exact.
    int4v kst[2][kCpt], vst[2][kCpt];  // [set][chunk]
    auto load = [&](int kt, int set) {
      const int key0 = kt * kTile;
  #pragma unroll
      for (int p = 0; p < kCpt; ++p) {
        const int r = cr + kRowStep * p;
        kst[set][p] = __builtin_amdgcn_raw_buffer_load_b128(krsrc, ((key0 + r) * kD + cc * 8) * 2, 0, 0);
        if (VT_VEC) {
          const int off = key0 + cc * 8 < T ? (r * T + key0 + cc * 8) * 2 : kOutOfRange;
          vst[set][p] = __builtin_amdgcn_raw_buffer_load_b128(vrsrc, off, 0, 0);
        } else {
          half8 v;
  #pragma unroll
          for (int e = 0; e < 8; ++e) {
            const int key = key0 + cc * 8 + e;
            v[e] = key < T ? Vh[(size_t)r * T + key] : (half_t)0;
          }
          vst[set][p] = __builtin_bit_cast(int4v, v);
        }
      }
    };
    auto store = [&](int buf, int set) {
  #pragma unroll
      for (int p = 0; p < kCpt; ++p) {
        const int off = buf * kTileHalfs + chunk_offset(cr + kRowStep * p, cc);
        *reinterpret_cast<int4v*>(kbuf + off) = kst[set][p];
        *reinterpret_cast<int4v*>(vbuf + off) = vst[set][p];
      }
    };

    // natural K rows for S^T (keys krow(n), d = 16kk + 8g ..)
    int kOff[4];
  #pragma unroll
    for (int kk = 0; kk < 4; ++kk) kOff[kk] = chunk_offset(krow(n), 2 * kk + g);
    // V rows (keys krow(n) + 32 mh) from the V^T tile; K^T rows (d = n + 32 mh) from the K tile
    int vtOff[2][2], ktOff[2][2];
  #pragma unroll
    for (int mh = 0; mh < 2; ++mh)
  #pragma unroll
      for (int hi = 0; hi < 2; ++hi) {
        vtOff[mh][hi] = tr_offset(lane, true, mh, hi);
        ktOff[mh][hi] = tr_offset(lane, false, mh, hi);
      }

    float16v dq0 = {}, dq1 = {};
    load(0, 0);
    load(1, 1);
    store(0, 0);
    __builtin_amdgcn_s_waitcnt(kLdsDone);
    barrier();
    // Tile kt + 1 goes into LDS at the start of step kt (its buffer held
    // tile kt - 1, which every wave finished before the last barrier), so the
    // stores complete under the step's products; A/B on one MI355X against
    // storing at the step's end: 0.6 to 2.4 % faster over the whole backward,
    // outputs bit-identical.
    auto tile_step = [&](int kt, int buf) {
      store(buf ^ 1, buf ^ 1);
      load(kt + 2, buf);
      if (kt * kTile <= waveLast) {
        const half_t* kb = kbuf + buf * kTileHalfs;
        const half_t* vb = vbuf + buf * kTileHalfs;
        // S^T = K Q^T and dP^T = V dO^T: keys 0..31 (x0) and 32..63 (x1) of the tile
        float16v s0, s1, p0, p1;
  #pragma unroll
        for (int kk = 0; kk < 4; ++kk) {
          const half8 a0 = ld8(kb + kOff[kk]);
          const half8 a1 = ld8(kb + kOff[kk] + 32 * kRowHalfs);
          s0 = mfma(a0, qf[kk], kk == 0 ? float16v{} : s0);
          s1 = mfma(a1, qf[kk], kk == 0 ? float16v{} : s1);
          const half_t* vk = vb + 16 * kk * kRowHalfs;
          const half8 v0 = tr8(vk, vtOff[0][0], vtOff[0][1]);
          const half8 v1 = tr8(vk, vtOff[1][0], vtOff[1][1]);
          // the dP^T accumulators start at -D, so they end as dP^T - D
          p0 = mfma(v0, dof[kk], kk == 0 ? negD : p0);
          p1 = mfma(v1, dof[kk], kk == 0 ? negD : p1);
        }
        // the diagonal: key 64kt + 16(i/8) + 8g + i%8 (+32) is kept iff <= row
        if (kt * kTile + kTile - 1 > waveRow0) {
          const int lim = row - kt * kTile - 8 * g;
  #pragma unroll
          for (int i = 0; i < 16; ++i) {
            const int k = 16 * (i >> 3) + (i & 7);
            if (k > lim) s0[i] = -INFINITY;
            if (k + 32 > lim) s1[i] = -INFINITY;
          }
        }
        // P^T = 2^(S^T c - L), dS^T = P^T (dP^T - D)
  #pragma unroll
        for (int i = 0; i < 16; ++i) {
          s0[i] = __builtin_amdgcn_exp2f(fmaf(s0[i], c, negL)) * p0[i];
          s1[i] = __builtin_amdgcn_exp2f(fmaf(s1[i], c, negL)) * p1[i];
        }
        const half8 ds[4] = {pack8(s0, 0), pack8(s0, 1), pack8(s1, 0), pack8(s1, 1)};
        // dQ^T += K^T dS^T: d = n (dq0) and 32 + n (dq1), keys 16ck + 8g .. +7
  #pragma unroll
        for (int ck = 0; ck < 4; ++ck) {
          const half_t* kc = kb + 16 * ck * kRowHalfs;
          const half8 k0 = tr8(kc, ktOff[0][0], ktOff[0][1]);
          const half8 k1 = tr8(kc, ktOff[1][0], ktOff[1][1]);
          dq0 = mfma(k0, ds[ck], dq0);
          dq1 = mfma(k1, ds[ck], dq1);
        }
      }
      __builtin_amdgcn_s_waitcnt(kLdsDone);
      barrier();
    };
    for (int kt = 0; kt < nkt; kt += 2) {  // unrolled by two: the sets are fixed registers
      tile_step(kt, 0);
      if (kt + 1 < nkt) tile_step(kt + 1, 1);
    }

    // dQ = s * sum: accumulator element 4q + e of lane (n, g) is d = 8q + 4g + e
    if (live) {
      float* out = dQ + ((size_t)h * T + row) * kD + 4 * g;
  #pragma unroll
      for (int q = 0; q < 4; ++q) {
        const float4v a = {dq0[4 * q], dq0[4 * q + 1], dq0[4 * q + 2], dq0[4 * q + 3]};
        const float4v b = {dq1[4 * q], dq1[4 * q + 1], dq1[4 * q + 2], dq1[4 * q + 3]};
        *reinterpret_cast<float4v*>(out + 8 * q) = a * s;
        *reinterpret_cast<float4v*>(out + 32 + 8 * q) = b * s;
      }
    }
  };
  run(nBlocks - 1 - pair);
  if (PAIRED && pair != nBlocks - 1 - pair) run(pair);
}

// -------------------------------------------------------------------------
// Key launch: dK and dV^T of query head h's contribution.  Workgroup = NW
// waves x 32 keys of K/V head h / G.
// -------------------------------------------------------------------------
template <int NW, bool VT_VEC, bool PAIRED>
__global__ void __launch_bounds__(64 * NW, 8 / NW)
sattn_bwdk_kernel(const half_t* __restrict__ Q, const half_t* __restrict__ K,
                  const half_t* __restrict__ Vt, const half_t* __restrict__ dO,
                  const float* __restrict__ L, const float* __restrict__ D,
                  float* __restrict__ dKp, float* __restrict__ dVp, float c, float s, int T,
                  int Hq, int G, int nBlocks, int nPairs) {
  __shared__ __attribute__((aligned(16))) half_t smem[4 * kTileHalfs];
  __shared__ __attribute__((aligned(16))) float rowterms[2][2][kTile];  // [buf][L, D][query]
  half_t* const qbuf = smem;                    // Q tiles [2][64 queries][64], chunks swizzled
  half_t* const obuf = smem + 2 * kTileHalfs;   // dO tiles [2][64 queries][64], chunks swizzled

  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lane = tid & 63;
  const int n = lane & 31;
  const int g = lane >> 5;

  // K/V head first, then key blocks heaviest first (paired: heavy block p,
  // then light block nBlocks-1-p, so every workgroup carries the same causal
  // work), then the group's heads
  const int lid = xcd_order();
  const int kv = lid / (nPairs * G);
  const int rem = lid - kv * nPairs * G;
  const int pair = rem / G;
  const int h = kv * G + rem % G;
  auto run = [&](int blk) {
    const int key0 = blk * 32 * NW;
    const int waveKey0 = key0 + 32 * wave;
    const int key = waveKey0 + n;
    const bool live = key < T;
    const int ft = key0 / kTile;                  // first query tile (key0 is a multiple of 64)
    const int nt = (T + kTile - 1) / kTile;

    // K and V rows of the wave's keys as B operands (lane: key n, d = 16kk + 8g .. +7)
    half8 kf[4], vf[4];
    {
      const half_t* krow_p = K + ((size_t)kv * T + key) * kD + 8 * g;
      const half_t* vcol = Vt + (size_t)kv * kD * T + key;
  #pragma unroll
      for (int kk = 0; kk < 4; ++kk) {
        kf[kk] = live ? ld8(krow_p + 16 * kk) : half8{};
  #pragma unroll
        for (int e = 0; e < 8; ++e)
          vf[kk][e] = live ? vcol[(size_t)(16 * kk + 8 * g + e) * T] : (half_t)0;
      }
    }

    // Staging: thread t owns 16-byte chunks t, t + 64 NW, .. of the Q tile and
    // of the dO tile (row c/8, column chunk c%8); threads 0..63 the tile's L
    // and threads 64..127 its -D (rows past T read L = +inf and -D = 0, so
    // P = 0).
    constexpr int kCpt = 512 / (64 * NW), kRowStep = 8 * NW;  // chunks per thread, rows between them
    const int cr = tid >> 3, cc = tid & 7;
    const __amdgpu_buffer_rsrc_t qrsrc = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<half_t*>(Q + (size_t)h * T * kD), 0, T * kD * 2, kBufferWord3);
    const __amdgpu_buffer_rsrc_t orsrc = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<half_t*>(dO + (size_t)h * kD), 0, (T * Hq - h) * kD * 2, kBufferWord3);
    // Two register sets by tile parity, loads two tiles ahead (as in the query
    // launch); tiles past the end read as zeros and their row terms as L = +inf,
    // -D = 0.
    int4v qst[2][kCpt], ost[2][kCpt];  // [set][chunk]
    float rst[2] = {0.0f, 0.0f};
    auto load = [&](int it, int set) {
      const int q0 = it * kTile;
  #pragma unroll
      for (int p = 0; p < kCpt; ++p) {
        const int r = q0 + cr + kRowStep * p;
        qst[set][p] = __builtin_amdgcn_raw_buffer_load_b128(qrsrc, (r * kD + cc * 8) * 2, 0, 0);
        ost[set][p] = __builtin_amdgcn_raw_buffer_load_b128(
            orsrc, (int)(((unsigned)r * (unsigned)Hq * kD + cc * 8) * 2u), 0, 0);
      }
      if (tid < 2 * kTile) {
        const int q = q0 + (tid & (kTile - 1));
        const bool isL = tid < kTile;
        rst[set] = q < T ? (isL ? L[(size_t)h * T + q] : -D[(size_t)h * T + q]) : (isL ? INFINITY : 0.0f);
      }
    };
    auto store = [&](int buf, int set) {
  #pragma unroll
      for (int p = 0; p < kCpt; ++p) {
        const int off = buf * kTileHalfs + chunk_offset(cr + kRowStep * p, cc);
        *reinterpret_cast<int4v*>(qbuf + off) = qst[set][p];
        *reinterpret_cast<int4v*>(obuf + off) = ost[set][p];
      }
      if (tid < 2 * kTile) rowterms[buf][tid >> 6][tid & (kTile - 1)] = rst[set];
    };

    // natural Q / dO rows (queries krow(n), d = 16kk + 8g ..)
    int nOff[4];
  #pragma unroll
    for (int kk = 0; kk < 4; ++kk) nOff[kk] = chunk_offset(krow(n), 2 * kk + g);
    // Q^T / dO^T rows (d = n + 32 mh)
    int tOff[2][2];
  #pragma unroll
    for (int mh = 0; mh < 2; ++mh)
  #pragma unroll
      for (int hi = 0; hi < 2; ++hi) tOff[mh][hi] = tr_offset(lane, false, mh, hi);

    float16v dk0 = {}, dk1 = {}, dv0 = {}, dv1 = {};
    load(ft, 0);
    load(ft + 1, 1);
    store(0, 0);
    __builtin_amdgcn_s_waitcnt(kLdsDone);
    barrier();
    // tile it + 1 goes into LDS at the start of step it, as in the query launch
    auto tile_step = [&](int it, int buf) {
      store(buf ^ 1, buf ^ 1);
      load(it + 2, buf);
      if (it * kTile + kTile - 1 >= waveKey0) {
        const half_t* qb = qbuf + buf * kTileHalfs;
        const half_t* ob = obuf + buf * kTileHalfs;
        // -D of element i's query 16(i/8) + 8g + i%8 (+32 for x1): the dP
        // accumulators start there, so they end as dP - D
        const float* lt = rowterms[buf][0];
        const float* dt = rowterms[buf][1];
        float16v nd0, nd1;
  #pragma unroll
        for (int b = 0; b < 4; ++b) {
          const float4v d0 = *reinterpret_cast<const float4v*>(dt + 16 * b + 8 * g);
          const float4v d1 = *reinterpret_cast<const float4v*>(dt + 16 * b + 8 * g + 4);
  #pragma unroll
          for (int e = 0; e < 4; ++e) {
            float16v& nd = b < 2 ? nd0 : nd1;
            nd[8 * (b & 1) + e] = d0[e];
            nd[8 * (b & 1) + 4 + e] = d1[e];
          }
        }
        // S = Q K^T and dP = dO V^T: queries 0..31 (x0) and 32..63 (x1) of the tile
        float16v s0, s1, p0, p1;
  #pragma unroll
        for (int kk = 0; kk < 4; ++kk) {
          const half8 a0 = ld8(qb + nOff[kk]);
          const half8 a1 = ld8(qb + nOff[kk] + 32 * kRowHalfs);
          s0 = mfma(a0, kf[kk], kk == 0 ? float16v{} : s0);
          s1 = mfma(a1, kf[kk], kk == 0 ? float16v{} : s1);
          const half8 b0 = ld8(ob + nOff[kk]);
          const half8 b1 = ld8(ob + nOff[kk] + 32 * kRowHalfs);
          p0 = mfma(b0, vf[kk], kk == 0 ? nd0 : p0);
          p1 = mfma(b1, vf[kk], kk == 0 ? nd1 : p1);
        }
        // the diagonal: query 64it + 16(i/8) + 8g + i%8 (+32) is kept iff >= key
        if (it * kTile < waveKey0 + 31) {
          const int lim = key - it * kTile - 8 * g;
  #pragma unroll
          for (int i = 0; i < 16; ++i) {
            const int q = 16 * (i >> 3) + (i & 7);
            if (q < lim) s0[i] = -INFINITY;
            if (q + 32 < lim) s1[i] = -INFINITY;
          }
        }
        // P = 2^(S c - L) and dS = P (dP - D), eight queries at a time: block
        // b holds queries 16b + 8g .. +7 of the tile (elements 8(b%2) .. of x(b/2))
        half8 pb[4], db[4];
  #pragma unroll
        for (int b = 0; b < 4; ++b) {
          const int q = 16 * b + 8 * g;
          const float4v l0 = *reinterpret_cast<const float4v*>(lt + q);
          const float4v l1 = *reinterpret_cast<const float4v*>(lt + q + 4);
  #pragma unroll
          for (int e = 0; e < 8; ++e) {
            const int i = 8 * (b & 1) + e;
            const float sv = b < 2 ? s0[i] : s1[i];
            const float pv = b < 2 ? p0[i] : p1[i];
            const float lv = e < 4 ? l0[e] : l1[e - 4];
            const float P = __builtin_amdgcn_exp2f(fmaf(sv, c, -lv));
            pb[b][e] = (half_t)P;
            db[b][e] = (half_t)(P * pv);
          }
        }
        // dV^T += dO^T P and dK^T += Q^T dS: d = n (x0) and 32 + n (x1),
        // queries 16ck + 8g .. +7
  #pragma unroll
        for (int ck = 0; ck < 4; ++ck) {
          const half_t* oc = ob + 16 * ck * kRowHalfs;
          const half_t* qc = qb + 16 * ck * kRowHalfs;
          const half8 o0 = tr8(oc, tOff[0][0], tOff[0][1]);
          const half8 o1 = tr8(oc, tOff[1][0], tOff[1][1]);
          dv0 = mfma(o0, pb[ck], dv0);
          dv1 = mfma(o1, pb[ck], dv1);
          const half8 q0 = tr8(qc, tOff[0][0], tOff[0][1]);
          const half8 q1 = tr8(qc, tOff[1][0], tOff[1][1]);
          dk0 = mfma(q0, db[ck], dk0);
          dk1 = mfma(q1, db[ck], dk1);
        }
      }
      __builtin_amdgcn_s_waitcnt(kLdsDone);
      barrier();
    };
    for (int it = ft; it < nt; it += 2) {  // unrolled by two: the sets are fixed registers
      tile_step(it, 0);
      if (it + 1 < nt) tile_step(it + 1, 1);
    }

    // accumulator element 4q + e of lane (n, g) is d = 8q + 4g + e of key n
    if (live) {
      float* kout = dKp + ((size_t)h * T + key) * kD + 4 * g;
  #pragma unroll
      for (int q = 0; q < 4; ++q) {
        const float4v a = {dk0[4 * q], dk0[4 * q + 1], dk0[4 * q + 2], dk0[4 * q + 3]};
        const float4v b = {dk1[4 * q], dk1[4 * q + 1], dk1[4 * q + 2], dk1[4 * q + 3]};
        *reinterpret_cast<float4v*>(kout + 8 * q) = a * s;
        *reinterpret_cast<float4v*>(kout + 32 + 8 * q) = b * s;
      }
      float* vout = dVp + (size_t)h * kD * T + key;
  #pragma unroll
      for (int i = 0; i < 16; ++i) {
        const int d = 8 * (i >> 2) + 4 * g + (i & 3);
        vout[(size_t)d * T] = dv0[i];
        vout[(size_t)(d + 32) * T] = dv1[i];
      }
    }
  };
  run(pair);
  if (PAIRED && pair != nBlocks - 1 - pair) run(nBlocks - 1 - pair);
}

// -------------------------------------------------------------------------
// Launches for grids too small to fill the chip: a workgroup of four waves
// takes one 32-row block (queries, or keys) of one head and its waves walk
// the block's tiles round-robin (tile w, w + 4, ...), each staging its own
// tiles in a private LDS region (coalesced loads, no barrier in the loop).
// The four partial accumulators are summed in wave order at the end, so the
// result is deterministic.  The tile bodies are those of the launches above.
// -------------------------------------------------------------------------
constexpr int kSW = 4;  // waves per workgroup of the split launches
constexpr int kPartRow = kD + 4;  // floats per row of a partial in LDS

// A wave's 32 x 64 binary32 partial, row-major with kPartRow-float rows, from
// its accumulators: element 4q + e of lane (n, g) is column 8q + 4g + e of row
// n (a1: column + 32).
__device__ __forceinline__ void store_partial_rows(float* part, const float16v& a0,
                                                   const float16v& a1, int lane) {
  const int n = lane & 31, g = lane >> 5;
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const float4v a = {a0[4 * q], a0[4 * q + 1], a0[4 * q + 2], a0[4 * q + 3]};
    const float4v b = {a1[4 * q], a1[4 * q + 1], a1[4 * q + 2], a1[4 * q + 3]};
    *reinterpret_cast<float4v*>(part + n * kPartRow + 8 * q + 4 * g) = a;
    *reinterpret_cast<float4v*>(part + n * kPartRow + 32 + 8 * q + 4 * g) = b;
  }
}

// Rows 8 wave .. 8 wave + 7 of the sum of the kSW partials (in wave order),
// times s, to out rows row0 + r < T: lane l takes row 8 wave + l/8, columns
// 8(l%8) .. +7.
template <typename Region>
__device__ __forceinline__ void sum_rows_out(const Region& region, float* out, int row0, int T,
                                             float s, int wave, int lane) {
  const int r = 8 * wave + (lane >> 3), ch = lane & 7;
  const float* p0 = reinterpret_cast<const float*>(region[0]) + r * kPartRow + 8 * ch;
  float4v a = *reinterpret_cast<const float4v*>(p0);
  float4v b = *reinterpret_cast<const float4v*>(p0 + 4);
#pragma unroll
  for (int w = 1; w < kSW; ++w) {
    const float* pw = reinterpret_cast<const float*>(region[w]) + r * kPartRow + 8 * ch;
    a += *reinterpret_cast<const float4v*>(pw);
    b += *reinterpret_cast<const float4v*>(pw + 4);
  }
  if (row0 + r < T) {
    float* const o = out + (size_t)(row0 + r) * kD + 8 * ch;
    *reinterpret_cast<float4v*>(o) = a * s;
    *reinterpret_cast<float4v*>(o + 4) = b * s;
  }
}

// DMA (V^T chunks whole 16-byte loads only): each wave double-buffers its
// tiles in LDS with direct-to-LDS loads, one workgroup per compute unit;
// otherwise the next tile waits in registers (PREFETCH) or is loaded at the
// start of its turn, two workgroups per unit.
template <bool VT_VEC, bool PREFETCH, bool DMA>
__global__ void __launch_bounds__(64 * kSW, DMA ? 1 : 2)
sattn_bwdq_split_kernel(const half_t* __restrict__ Q, const half_t* __restrict__ K,
                        const half_t* __restrict__ Vt, const half_t* __restrict__ O,
                        const half_t* __restrict__ dO, const float* __restrict__ L,
                        float* __restrict__ dQ, float* __restrict__ D, float c, float s, int T,
                        int Hq, int G, int nBlocks, int nPairs, int pairsPerXcd) {
  // wave w's region: its K tile and V^T tile (with DMA two such pairs);
  // afterwards its partial dQ
  static_assert(!DMA || VT_VEC, "LDS loads need whole 16-byte V^T chunks");
  __shared__ __attribute__((aligned(16))) half_t region[kSW][(DMA ? 4 : 2) * kTileHalfs];
  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lane = tid & 63;
  const int n = lane & 31;
  const int g = lane >> 5;

  // heavy query block n-1-j, light block j (see split_unit)
  int kv, h, jp;
  bool lightUnit;
  if (!split_unit(nBlocks, G, nPairs, pairsPerXcd, kv, h, jp, lightUnit)) return;
  const int blk = lightUnit ? jp : nBlocks - 1 - jp;
  const int row0 = 32 * blk;
  const int row = row0 + n;
  const bool live = row < T;
  const int nkt = min(T - 1, row0 + 31) / kTile + 1;  // key tiles up to the diagonal

  half8 qf[4], dof[4];
  float dpart = 0.0f;
  {
    const half_t* qrow = Q + ((size_t)h * T + row) * kD + 8 * g;
    const size_t tok = (size_t)row * Hq * kD + (size_t)h * kD + 8 * g;
  #pragma unroll
    for (int kk = 0; kk < 4; ++kk) {
      const half8 z = {};
      qf[kk] = live ? ld8(qrow + 16 * kk) : z;
      dof[kk] = live ? *reinterpret_cast<const half8*>(dO + tok + 16 * kk) : z;
      const half8 of = live ? *reinterpret_cast<const half8*>(O + tok + 16 * kk) : z;
  #pragma unroll
      for (int e = 0; e < 8; ++e) dpart = fmaf((float)dof[kk][e], (float)of[e], dpart);
    }
  }
  const float Drow = dpart + xlane(dpart, (lane ^ 32) << 2);
  const float negL = live ? -L[(size_t)h * T + row] : 0.0f;
  float16v negD;
  #pragma unroll
  for (int i = 0; i < 16; ++i) negD[i] = -Drow;
  if (wave == 0 && live && g == 0) D[(size_t)h * T + row] = Drow;

  // Staging: lane l owns chunk l + 64 i (i < 8) of each tile: row l/8 + 8i,
  // chunk l%8 (tiles past the end and V^T chunks past T read as zeros).
  half_t* const kb = region[wave];
  half_t* const vb = region[wave] + kTileHalfs;
  const int sr = lane >> 3, sc = lane & 7;
  const __amdgpu_buffer_rsrc_t krsrc = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<half_t*>(K + (size_t)kv * T * kD), 0, T * kD * 2, kBufferWord3);
  const half_t* Vh = Vt + (size_t)kv * kD * T;
  const __amdgpu_buffer_rsrc_t vrsrc =
      __builtin_amdgcn_make_buffer_rsrc(const_cast<half_t*>(Vh), 0, kD * T * 2, kBufferWord3);
  int4v st[16];  // the next tile: K chunks 0..7, V^T chunks 8..15
  auto load = [&](int kt) {
    const int key0 = kt * kTile;
  #pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int r = sr + 8 * i;
      st[i] = __builtin_amdgcn_raw_buffer_load_b128(krsrc, ((key0 + r) * kD + sc * 8) * 2, 0, 0);
      if (VT_VEC) {
        const int off = key0 + sc * 8 < T ? (r * T + key0 + sc * 8) * 2 : kOutOfRange;
        st[8 + i] = __builtin_amdgcn_raw_buffer_load_b128(vrsrc, off, 0, 0);
      } else {
        half8 v;
  #pragma unroll
        for (int e = 0; e < 8; ++e) {
          const int key = key0 + sc * 8 + e;
          v[e] = key < T ? Vh[(size_t)r * T + key] : (half_t)0;
        }
        st[8 + i] = __builtin_bit_cast(int4v, v);
      }
    }
  };
  auto store = [&]() {
  #pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int off = chunk_offset(sr + 8 * i, sc);
      *reinterpret_cast<int4v*>(kb + off) = st[i];
      *reinterpret_cast<int4v*>(vb + off) = st[8 + i];
    }
  };

  int kOff[4];
  #pragma unroll
  for (int kk = 0; kk < 4; ++kk) kOff[kk] = chunk_offset(krow(n), 2 * kk + g);
  int vtOff[2][2], ktOff[2][2];
  #pragma unroll
  for (int mh = 0; mh < 2; ++mh)
  #pragma unroll
    for (int hi = 0; hi < 2; ++hi) {
      vtOff[mh][hi] = tr_offset(lane, true, mh, hi);
      ktOff[mh][hi] = tr_offset(lane, false, mh, hi);
    }

  float16v dq0 = {}, dq1 = {};
  // One key tile: S^T and dP^T (started at -D), P, dS, then dQ^T.
  auto tile = [&](const half_t* kb, const half_t* vb, int kt) {
    float16v s0, s1, p0, p1;
  #pragma unroll
    for (int kk = 0; kk < 4; ++kk) {
      s0 = mfma(ld8(kb + kOff[kk]), qf[kk], kk == 0 ? float16v{} : s0);
      s1 = mfma(ld8(kb + kOff[kk] + 32 * kRowHalfs), qf[kk], kk == 0 ? float16v{} : s1);
      const half_t* vk = vb + 16 * kk * kRowHalfs;
      p0 = mfma(tr8(vk, vtOff[0][0], vtOff[0][1]), dof[kk], kk == 0 ? negD : p0);
      p1 = mfma(tr8(vk, vtOff[1][0], vtOff[1][1]), dof[kk], kk == 0 ? negD : p1);
    }
    if (kt * kTile + kTile - 1 > row0) {
      const int lim = row - kt * kTile - 8 * g;
  #pragma unroll
      for (int i = 0; i < 16; ++i) {
        const int k = 16 * (i >> 3) + (i & 7);
        if (k > lim) s0[i] = -INFINITY;
        if (k + 32 > lim) s1[i] = -INFINITY;
      }
    }
  #pragma unroll
    for (int i = 0; i < 16; ++i) {
      s0[i] = __builtin_amdgcn_exp2f(fmaf(s0[i], c, negL)) * p0[i];
      s1[i] = __builtin_amdgcn_exp2f(fmaf(s1[i], c, negL)) * p1[i];
    }
    const half8 ds[4] = {pack8(s0, 0), pack8(s0, 1), pack8(s1, 0), pack8(s1, 1)};
  #pragma unroll
    for (int ck = 0; ck < 4; ++ck) {
      const half_t* kc = kb + 16 * ck * kRowHalfs;
      dq0 = mfma(tr8(kc, ktOff[0][0], ktOff[0][1]), ds[ck], dq0);
      dq1 = mfma(tr8(kc, ktOff[1][0], ktOff[1][1]), ds[ck], dq1);
    }
  };

  int kt = wave;
  if constexpr (DMA) {
    // Pair A and pair B: a K tile and a V^T tile each.  Piece i (1 KiB) of a
    // tile holds its rows 8i .. 8i+7, lane l's 16 bytes at row 8i + l/8, slot
    // l%8, which holds chunk (l%8) ^ swz(row) (swz depends on i only through
    // i % 2).  K rows past T and V^T chunks past T (T % 8 == 0) read as zeros.
    const int pr = lane >> 3;
    int pc[2];
  #pragma unroll
    for (int e = 0; e < 2; ++e) pc[e] = (lane & 7) ^ sattn_lds::swz(8 * e + pr);
    const int4v kdesc = sattn_lds::raw_desc(K + (size_t)kv * T * kD, (unsigned)T * kD * 2);
    const int4v vdesc = sattn_lds::raw_desc(Vh, (unsigned)kD * T * 2);
    half_t* const kA = region[wave];
    half_t* const vA = kA + kTileHalfs;
    half_t* const kB = kA + 2 * kTileHalfs;
    half_t* const vB = kA + 3 * kTileHalfs;
    constexpr int kLoads = 16;  // direct-to-LDS loads per pair
    // The wave's earlier reads of the pair have returned (the products
    // consumed them) before it is refilled.
    auto issue = [&](half_t* kd, half_t* vd, int t) {
      __builtin_amdgcn_s_waitcnt(kLdsDone);
      const unsigned key0 = (unsigned)t * kTile;
      const unsigned kl = sattn_lds::lds_addr(kd), vl = sattn_lds::lds_addr(vd);
  #pragma unroll
      for (int i = 0; i < 8; ++i) {
        const unsigned r = 8u * i + pr, ch = (unsigned)pc[i & 1];
        sattn_lds::lds_load16(kdesc, __builtin_amdgcn_readfirstlane(kl + 1024u * i),
                              ((key0 + r) * kD + ch * 8) * 2);
        const unsigned vByte = key0 + ch * 8 < (unsigned)T ? (r * (unsigned)T + key0 + ch * 8) * 2
                                                           : (unsigned)kOutOfRange;
        sattn_lds::lds_load16(vdesc, __builtin_amdgcn_readfirstlane(vl + 1024u * i), vByte);
      }
    };
    auto wait_pair = [&](bool keepNext) {
      if (keepNext) __builtin_amdgcn_s_waitcnt(sattn_lds::vmcnt_only(kLoads));
      else __builtin_amdgcn_s_waitcnt(sattn_lds::vmcnt_only(0));
      asm volatile("" ::: "memory");
    };
    if (kt < nkt) issue(kA, vA, kt);
    if (kt + kSW < nkt) issue(kB, vB, kt + kSW);
    while (kt < nkt) {
      wait_pair(kt + kSW < nkt);
      tile(kA, vA, kt);
      if (kt + 2 * kSW < nkt) issue(kA, vA, kt + 2 * kSW);
      kt += kSW;
      if (kt >= nkt) break;
      wait_pair(kt + kSW < nkt);
      tile(kB, vB, kt);
      if (kt + 2 * kSW < nkt) issue(kB, vB, kt + 2 * kSW);
      kt += kSW;
    }
  } else {
    if (PREFETCH && kt < nkt) load(kt);
    while (kt < nkt) {
      // the previous tile's reads were consumed by the products
      if (!PREFETCH) load(kt);
      store();
      __builtin_amdgcn_s_waitcnt(kLdsDone);
      const int kn = kt + kSW;
      if (PREFETCH && kn < nkt) load(kn);
      tile(kb, vb, kt);
      kt = kn;
    }
  }

  // Sum the four partials in wave order: every wave leaves its partial in its
  // region (row-major), then wave w sums rows 8w .. 8w+7 and writes them as
  // whole 256-byte rows (eight lanes a row).
  store_partial_rows(reinterpret_cast<float*>(region[wave]), dq0, dq1, lane);
  __syncthreads();
  sum_rows_out(region, dQ + (size_t)h * T * kD, 32 * blk, T, s, wave, lane);
}

// DMA: each wave double-buffers its tiles in LDS with direct-to-LDS loads
// (the tile four further along lands while one is computed), one workgroup
// per compute unit; otherwise the tile is loaded into registers at the start
// of its turn (PREFETCH: one turn ahead) and stored, two workgroups per unit.
template <bool PREFETCH, bool DMA>
__global__ void __launch_bounds__(64 * kSW, DMA ? 1 : 2)
sattn_bwdk_split_kernel(const half_t* __restrict__ Q, const half_t* __restrict__ K,
                        const half_t* __restrict__ Vt, const half_t* __restrict__ dO,
                        const float* __restrict__ L, const float* __restrict__ D,
                        float* __restrict__ dKp, float* __restrict__ dVp, float c, float s, int T,
                        int Hq, int G, int nBlocks, int nPairs, int pairsPerXcd) {
  // wave w's region: its Q tile, dO tile and the tile's L and -D (with DMA:
  // two such sets, and D instead of -D); afterwards its partial dK^T and dV^T
  constexpr int kSet = 2 * kTileHalfs * 2 + 2 * kTile * 4;  // bytes
  constexpr int kRegion = DMA ? 2 * kSet : kSet;
  __shared__ __attribute__((aligned(16))) char region[kSW][kRegion];
  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lane = tid & 63;
  const int n = lane & 31;
  const int g = lane >> 5;

  // heavy key block j (every later query sees it), light block n-1-j (see
  // split_unit)
  int kv, h, jp;
  bool lightUnit;
  if (!split_unit(nBlocks, G, nPairs, pairsPerXcd, kv, h, jp, lightUnit)) return;
  const int blk = lightUnit ? nBlocks - 1 - jp : jp;
  const int key0 = 32 * blk;
  const int key = key0 + n;
  const bool live = key < T;
  const int ft = key0 / kTile;  // the first query tile holding a query >= key0
  const int nt = (T + kTile - 1) / kTile;

  half8 kf[4], vf[4];
  {
    const half_t* krow_p = K + ((size_t)kv * T + key) * kD + 8 * g;
    const half_t* vcol = Vt + (size_t)kv * kD * T + key;
  #pragma unroll
    for (int kk = 0; kk < 4; ++kk) {
      kf[kk] = live ? ld8(krow_p + 16 * kk) : half8{};
  #pragma unroll
      for (int e = 0; e < 8; ++e) vf[kk][e] = live ? vcol[(size_t)(16 * kk + 8 * g + e) * T] : (half_t)0;
    }
  }

  half_t* const qb = reinterpret_cast<half_t*>(region[wave]);
  half_t* const ob = qb + kTileHalfs;
  float* const lt = reinterpret_cast<float*>(ob + kTileHalfs);  // [L][64], then [-D][64]
  const int sr = lane >> 3, sc = lane & 7;
  const __amdgpu_buffer_rsrc_t qrsrc = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<half_t*>(Q + (size_t)h * T * kD), 0, T * kD * 2, kBufferWord3);
  const __amdgpu_buffer_rsrc_t orsrc = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<half_t*>(dO + (size_t)h * kD), 0, (T * Hq - h) * kD * 2, kBufferWord3);
  int4v st[16];  // the next tile: Q chunks 0..7, dO chunks 8..15
  float rl = 0.0f, rd = 0.0f;
  auto load = [&](int it) {
    const int q0 = it * kTile;
  #pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int r = q0 + sr + 8 * i;
      st[i] = __builtin_amdgcn_raw_buffer_load_b128(qrsrc, (r * kD + sc * 8) * 2, 0, 0);
      st[8 + i] = __builtin_amdgcn_raw_buffer_load_b128(
          orsrc, (int)(((unsigned)r * (unsigned)Hq * kD + sc * 8) * 2u), 0, 0);
    }
    const int q = q0 + lane;  // queries past T: L = +inf and -D = 0, so P = 0
    rl = q < T ? L[(size_t)h * T + q] : INFINITY;
    rd = q < T ? -D[(size_t)h * T + q] : 0.0f;
  };
  auto store = [&]() {
  #pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int off = chunk_offset(sr + 8 * i, sc);
      *reinterpret_cast<int4v*>(qb + off) = st[i];
      *reinterpret_cast<int4v*>(ob + off) = st[8 + i];
    }
    lt[lane] = rl;
    lt[kTile + lane] = rd;
  };

  int nOff[4];
  #pragma unroll
  for (int kk = 0; kk < 4; ++kk) nOff[kk] = chunk_offset(krow(n), 2 * kk + g);
  int tOff[2][2];
  #pragma unroll
  for (int mh = 0; mh < 2; ++mh)
  #pragma unroll
    for (int hi = 0; hi < 2; ++hi) tOff[mh][hi] = tr_offset(lane, false, mh, hi);

  float16v dk0 = {}, dk1 = {}, dv0 = {}, dv1 = {};
  // One query tile: S, dP (started at -D), P and dS, then dV^T and dK^T.
  // With DMA the set holds D (negated here) and, for queries past T, L = 0:
  // their Q and dO rows are zeros, so P = 1 there meets dP - D = 0 and a zero
  // dO row, and adds nothing.
  auto tile = [&](const half_t* qb, const half_t* ob, const float* lt, int it) {
    const float* const dt = lt + kTile;
    float16v nd0, nd1;
  #pragma unroll
    for (int b = 0; b < 4; ++b) {
      const float4v d0 = *reinterpret_cast<const float4v*>(dt + 16 * b + 8 * g);
      const float4v d1 = *reinterpret_cast<const float4v*>(dt + 16 * b + 8 * g + 4);
  #pragma unroll
      for (int e = 0; e < 4; ++e) {
        float16v& nd = b < 2 ? nd0 : nd1;
        nd[8 * (b & 1) + e] = DMA ? -d0[e] : d0[e];
        nd[8 * (b & 1) + 4 + e] = DMA ? -d1[e] : d1[e];
      }
    }
    float16v s0, s1, p0, p1;
  #pragma unroll
    for (int kk = 0; kk < 4; ++kk) {
      s0 = mfma(ld8(qb + nOff[kk]), kf[kk], kk == 0 ? float16v{} : s0);
      s1 = mfma(ld8(qb + nOff[kk] + 32 * kRowHalfs), kf[kk], kk == 0 ? float16v{} : s1);
      p0 = mfma(ld8(ob + nOff[kk]), vf[kk], kk == 0 ? nd0 : p0);
      p1 = mfma(ld8(ob + nOff[kk] + 32 * kRowHalfs), vf[kk], kk == 0 ? nd1 : p1);
    }
    if (it * kTile < key0 + 31) {
      const int lim = key - it * kTile - 8 * g;
  #pragma unroll
      for (int i = 0; i < 16; ++i) {
        const int q = 16 * (i >> 3) + (i & 7);
        if (q < lim) s0[i] = -INFINITY;
        if (q + 32 < lim) s1[i] = -INFINITY;
      }
    }
    half8 pb[4], db[4];
  #pragma unroll
    for (int b = 0; b < 4; ++b) {
      const int q = 16 * b + 8 * g;
      const float4v l0 = *reinterpret_cast<const float4v*>(lt + q);
      const float4v l1 = *reinterpret_cast<const float4v*>(lt + q + 4);
  #pragma unroll
      for (int e = 0; e < 8; ++e) {
        const int i = 8 * (b & 1) + e;
        const float sv = b < 2 ? s0[i] : s1[i];
        const float pv = b < 2 ? p0[i] : p1[i];
        const float lv = e < 4 ? l0[e] : l1[e - 4];
        const float P = __builtin_amdgcn_exp2f(fmaf(sv, c, -lv));
        pb[b][e] = (half_t)P;
        db[b][e] = (half_t)(P * pv);
      }
    }
  #pragma unroll
    for (int ck = 0; ck < 4; ++ck) {
      const half_t* oc = ob + 16 * ck * kRowHalfs;
      const half_t* qc = qb + 16 * ck * kRowHalfs;
      dv0 = mfma(tr8(oc, tOff[0][0], tOff[0][1]), pb[ck], dv0);
      dv1 = mfma(tr8(oc, tOff[1][0], tOff[1][1]), pb[ck], dv1);
      dk0 = mfma(tr8(qc, tOff[0][0], tOff[0][1]), db[ck], dk0);
      dk1 = mfma(tr8(qc, tOff[1][0], tOff[1][1]), db[ck], dk1);
    }
  };

  int it = ft + wave;
  if constexpr (DMA) {
    // Set A and set B: Q tile, dO tile, L, D.  Piece i (1 KiB) of a tile
    // holds its rows 8i .. 8i+7, lane l's 16 bytes at row 8i + l/8, slot
    // l%8, which holds chunk (l%8) ^ swz(row) (swz depends on i only through
    // i % 2); L and D are one dword a lane.  Rows past T read as zeros.
    const int pr = lane >> 3;
    int pc[2];
  #pragma unroll
    for (int e = 0; e < 2; ++e) pc[e] = (lane & 7) ^ sattn_lds::swz(8 * e + pr);
    const int4v qdesc = sattn_lds::raw_desc(Q + (size_t)h * T * kD, (unsigned)T * kD * 2);
    const int4v odesc = sattn_lds::raw_desc(dO + (size_t)h * kD, (unsigned)(T * Hq - h) * kD * 2);
    const int4v ldesc = sattn_lds::raw_desc(L + (size_t)h * T, (unsigned)T * 4);
    const int4v ddesc = sattn_lds::raw_desc(D + (size_t)h * T, (unsigned)T * 4);
    char* const setA = region[wave];
    char* const setB = region[wave] + kSet;
    constexpr int kLoads = 18;  // direct-to-LDS loads per set
    // The wave's earlier reads of the set have returned (the products
    // consumed them) before it is refilled.
    auto issue = [&](char* set, int t) {
      __builtin_amdgcn_s_waitcnt(kLdsDone);
      const unsigned q0 = (unsigned)t * kTile;
      const unsigned ql = sattn_lds::lds_addr(set), ol = ql + kTileHalfs * 2;
  #pragma unroll
      for (int i = 0; i < 8; ++i) {
        const unsigned r = q0 + 8u * i + pr, ch = (unsigned)pc[i & 1];
        sattn_lds::lds_load16(qdesc, __builtin_amdgcn_readfirstlane(ql + 1024u * i), (r * kD + ch * 8) * 2);
        sattn_lds::lds_load16(odesc, __builtin_amdgcn_readfirstlane(ol + 1024u * i),
                              (r * (unsigned)Hq * kD + ch * 8) * 2);
      }
      const unsigned ll = ol + kTileHalfs * 2;
      sattn_lds::lds_load4(ldesc, __builtin_amdgcn_readfirstlane(ll), (q0 + lane) * 4);
      sattn_lds::lds_load4(ddesc, __builtin_amdgcn_readfirstlane(ll + kTile * 4), (q0 + lane) * 4);
    };
    auto wait_set = [&](bool keepNext) {
      if (keepNext) __builtin_amdgcn_s_waitcnt(sattn_lds::vmcnt_only(kLoads));
      else __builtin_amdgcn_s_waitcnt(sattn_lds::vmcnt_only(0));
      asm volatile("" ::: "memory");
    };
    auto run = [&](const char* set, int t) {
      const half_t* q = reinterpret_cast<const half_t*>(set);
      tile(q, q + kTileHalfs, reinterpret_cast<const float*>(q + 2 * kTileHalfs), t);
    };
    if (it < nt) issue(setA, it);
    if (it + kSW < nt) issue(setB, it + kSW);
    while (it < nt) {
      wait_set(it + kSW < nt);
      run(setA, it);
      if (it + 2 * kSW < nt) issue(setA, it + 2 * kSW);
      it += kSW;
      if (it >= nt) break;
      wait_set(it + kSW < nt);
      run(setB, it);
      if (it + 2 * kSW < nt) issue(setB, it + 2 * kSW);
      it += kSW;
    }
  } else {
    if (PREFETCH && it < nt) load(it);
    while (it < nt) {
      if (!PREFETCH) load(it);
      store();
      __builtin_amdgcn_s_waitcnt(kLdsDone);
      const int in = it + kSW;
      if (PREFETCH && in < nt) load(in);
      tile(qb, ob, lt, it);
      it = in;
    }
  }

  // Sum the four partials in wave order: every wave leaves its dK^T partial
  // (row-major) and its dV^T partial (accumulator order) in its region; wave
  // w then sums keys 8w .. 8w+7 of dK^T, written as whole 256-byte rows, and
  // d rows 16w .. 16w+15 of dV^T, written 32 consecutive keys a row.
  float* const part = reinterpret_cast<float*>(region[wave]);
  store_partial_rows(part, dk0, dk1, lane);
  float* const vpart = part + 32 * kPartRow;  // [32][64]: accumulator element i of dv0, dv1
  #pragma unroll
  for (int i = 0; i < 16; ++i) {
    vpart[i * 64 + lane] = dv0[i];
    vpart[(16 + i) * 64 + lane] = dv1[i];
  }
  __syncthreads();
  sum_rows_out(region, dKp + (size_t)h * T * kD, key0, T, s, wave, lane);
  // dV^T row d, key n: element 4(d%32/8) + d%4 of lane n + 32((d/4)%2), of dv1 if d >= 32
  const int kn = lane & 31;
  #pragma unroll
  for (int j = 0; j < 8; ++j) {
    const int d = 16 * wave + 2 * j + (lane >> 5);
    const int dd = d & 31;
    const int idx = (d >= 32 ? 16 : 0) + 4 * (dd >> 3) + (dd & 3);
    const int src = idx * 64 + kn + 32 * ((dd >> 2) & 1);
    float v = reinterpret_cast<const float*>(region[0])[32 * kPartRow + src];
  #pragma unroll
    for (int w = 1; w < kSW; ++w) v += reinterpret_cast<const float*>(region[w])[32 * kPartRow + src];
    if (key0 + kn < T) dVp[(size_t)h * kD * T + (size_t)d * T + key0 + kn] = v;
  }
}

// -------------------------------------------------------------------------
// Grouped gradient reduction: out[kv][e] = sum over z = 0..G-1, in order, of
// planes[kv G + z][e], for the dK planes (blockIdx.z = 0) and the dV^T
// planes (blockIdx.z = 1); a thread owns four consecutive elements.
// -------------------------------------------------------------------------
__global__ void __launch_bounds__(256)
sattn_bwd_reduce_kernel(const float* __restrict__ kPlanes, const float* __restrict__ vPlanes,
                        float* __restrict__ dK, float* __restrict__ dVt, int planeQuads, int G) {
  const int e4 = blockIdx.x * 256 + threadIdx.x;
  if (e4 >= planeQuads) return;
  const int kv = blockIdx.y;
  const float* src = (blockIdx.z == 0 ? kPlanes : vPlanes) + (size_t)kv * G * planeQuads * 4;
  float* dst = (blockIdx.z == 0 ? dK : dVt) + (size_t)kv * planeQuads * 4;
  float4v acc = *reinterpret_cast<const float4v*>(src + (size_t)e4 * 4);
  for (int z = 1; z < G; ++z)
    acc += *reinterpret_cast<const float4v*>(src + ((size_t)z * planeQuads + e4) * 4);
  *reinterpret_cast<float4v*>(dst + (size_t)e4 * 4) = acc;
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

// Launch shape.  Eight-wave workgroups (one per compute unit) stage each tile
// once for 256 rows and run a heavy block, then its light partner (blocks b
// and n-1-b), so every workgroup carries the same causal work; they are used
// when that grid still gives each of the 256 compute units a workgroup.
// Below that, when even the four-wave grid of 128-row blocks would hold fewer
// than two workgroups per compute unit, the split launches run (32-row
// blocks, their tiles dealt over four waves), so a block's walk is four times
// shorter.  Otherwise four-wave workgroups (two per compute unit) run, paired
// the same way when their halved grid still fills the compute units, and
// else one block each, heaviest first: idle units cost more than the
// imbalance.
constexpr long long kSplitBelow = 512;  // four-wave workgroups (128-row blocks x heads)
struct Shape {
  int nw, nBlocks, nPairs;
  bool paired, split;
};
Shape launch_shape(int T, int Hq) {
  const int n8 = (T + 255) / 256, n4 = (T + 127) / 128;
  if (n8 > 1 && (long long)((n8 + 1) / 2) * Hq >= 256) return {8, n8, (n8 + 1) / 2, true, false};
  if ((long long)n4 * Hq < kSplitBelow) {
    const int n = (T + 31) / 32;
    return {kSW, n, n, false, true};
  }
  const bool paired = n4 > 1 && (long long)((n4 + 1) / 2) * Hq >= 256;
  return {4, n4, paired ? (n4 + 1) / 2 : n4, paired, false};
}

// The split launches' grid: heavy/light pairs of 32-row blocks over all
// query heads, padded so each XCD takes a whole run of pairs (split_unit).
struct SplitGrid {
  int nPairs, pairsPerXcd;
  unsigned grid, units;
};
SplitGrid split_grid(int nBlocks, int Hq) {
  const int nPairs = (nBlocks + 1) / 2 * Hq;
  const int perXcd = (nPairs + kXcds - 1) / kXcds;
  return {nPairs, perXcd, (unsigned)perXcd * 2u * (unsigned)kXcds, (unsigned)nBlocks * (unsigned)Hq};
}

void launch_query(const half_t* Q, const half_t* K, const half_t* Vt, const half_t* O,
                  const half_t* dO, const float* L, float* dQ, float* D, float c, float s, int T,
                  int Hq, int Hkv, hipStream_t stream) {
  const Shape sh = launch_shape(T, Hq);
  const dim3 grid((unsigned)sh.nPairs * (unsigned)Hq);
  const int G = Hq / Hkv;
  const bool vec = T % 8 == 0;
  if (sh.split) {
    // direct-to-LDS double buffering (one workgroup per CU) when the blocks
    // fit the chip at once and V^T comes in whole 16-byte chunks
    const SplitGrid sg = split_grid(sh.nBlocks, Hq);
    auto sk = !vec                        ? sattn_bwdq_split_kernel<false, false, false>
              : sg.units <= (unsigned)kCus ? sattn_bwdq_split_kernel<true, false, true>
                                           : sattn_bwdq_split_kernel<true, true, false>;
    hipLaunchKernelGGL(sk, dim3(sg.grid), dim3(64 * kSW), 0, stream, Q, K, Vt, O, dO, L, dQ, D, c, s,
                       T, Hq, G, sh.nBlocks, sg.nPairs, sg.pairsPerXcd);
    return;
  }
  auto kernel = vec ? sattn_bwdq_kernel<8, true, true> : sattn_bwdq_kernel<8, false, true>;
  if (sh.nw == 4 && sh.paired)
    kernel = vec ? sattn_bwdq_kernel<4, true, true> : sattn_bwdq_kernel<4, false, true>;
  if (sh.nw == 4 && !sh.paired)
    kernel = vec ? sattn_bwdq_kernel<4, true, false> : sattn_bwdq_kernel<4, false, false>;
  hipLaunchKernelGGL(kernel, grid, dim3(64 * sh.nw), 0, stream, Q, K, Vt, O, dO, L, dQ, D, c, s, T,
                     Hq, G, sh.nBlocks, sh.nPairs);
}

void launch_key(const half_t* Q, const half_t* K, const half_t* Vt, const half_t* dO,
                const float* L, const float* D, float* dK, float* dVt, void* ws, float c, float s,
                int T, int Hq, int Hkv, hipStream_t stream) {
  const int G = Hq / Hkv;
  float* kp = G == 1 ? dK : static_cast<float*>(ws);
  float* vp = G == 1 ? dVt : static_cast<float*>(ws) + (size_t)Hq * T * kD;
  const Shape sh = launch_shape(T, Hq);
  const dim3 grid((unsigned)sh.nPairs * (unsigned)Hq);
  if (sh.split) {
    // direct-to-LDS double buffering (one workgroup per CU) when the blocks
    // fit the chip at once
    const SplitGrid sg = split_grid(sh.nBlocks, Hq);
    auto sk = sg.units <= (unsigned)kCus ? sattn_bwdk_split_kernel<false, true>
                                         : sattn_bwdk_split_kernel<false, false>;
    hipLaunchKernelGGL(sk, dim3(sg.grid), dim3(64 * kSW), 0, stream, Q, K, Vt, dO, L, D, kp, vp, c, s,
                       T, Hq, G, sh.nBlocks, sg.nPairs, sg.pairsPerXcd);
  } else {
    auto kernel = sattn_bwdk_kernel<8, true, true>;
    if (sh.nw == 4) kernel = sh.paired ? sattn_bwdk_kernel<4, true, true> : sattn_bwdk_kernel<4, true, false>;
    hipLaunchKernelGGL(kernel, grid, dim3(64 * sh.nw), 0, stream, Q, K, Vt, dO, L, D, kp, vp, c, s, T,
                       Hq, G, sh.nBlocks, sh.nPairs);
  }
  if (G > 1) {
    const int planeQuads = T * kD / 4;
    const dim3 rgrid((unsigned)((planeQuads + 255) / 256), (unsigned)Hkv, 2u);
    hipLaunchKernelGGL(sattn_bwd_reduce_kernel, rgrid, dim3(256), 0, stream, kp, vp, dK, dVt,
                       planeQuads, G);
  }
}

// sattn_bwd_key_noalloc's workspace: one static region per GPU, loaded with
// the library's code object.  In host code `scratch` names a host-side stand-in,
// not the device region: its device address is taken with
// hipGetSymbolAddress, once per device, and only that address is passed on.
constexpr unsigned long long kScratchBytes = SATTN_BWD_NOALLOC_MAX_BYTES;
__device__ __align__(256) float scratch[kScratchBytes / sizeof(float)];
std::atomic<float*> g_scratch_ptr[kMaxDevices];

// The current device's address of `scratch` (the device must be current), or
// NULL if the runtime cannot give it.
float* scratch_address() {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0) return nullptr;
  if (dev < kMaxDevices) {
    float* p = g_scratch_ptr[dev].load(std::memory_order_acquire);
    if (p) return p;
  }
  void* ptr = nullptr;
  if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)) != hipSuccess || ptr == nullptr) return nullptr;
  if (dev < kMaxDevices) g_scratch_ptr[dev].store(static_cast<float*>(ptr), std::memory_order_release);
  return static_cast<float*>(ptr);
}

}  // namespace

extern "C" int sattn_bwd_key_noalloc(const void* Q, const void* K, const void* Vt, const void* dO,
                                     const float* L, const float* D, float* dK, float* dVt,
                                     float c, float s, int T, int Hq, int Hkv, void* stream) {
  const int st = sattn_bwd_key_noalloc_check(Q, K, Vt, dO, L, D, dK, dVt, c, s, T, Hq, Hkv,
                                             kScratchBytes);
  if (st != SATTN_OK) return st;
  const int dst = check_device();
  if (dst != SATTN_OK) return dst;
  float* ws = nullptr;
  if (sattn_bwd_workspace_bytes(T, Hq, Hkv) > 0) {
    ws = scratch_address();
    if (ws == nullptr) return SATTN_ERR_DEVICE;
  }
  launch_key(static_cast<const half_t*>(Q), static_cast<const half_t*>(K),
             static_cast<const half_t*>(Vt), static_cast<const half_t*>(dO), L, D, dK, dVt, ws,
             c, s, T, Hq, Hkv, static_cast<hipStream_t>(stream));
  return hipGetLastError() == hipSuccess ? SATTN_OK : SATTN_ERR_LAUNCH;
}

extern "C" int sattn_bwd_query(const void* Q, const void* K, const void* Vt, const void* O,
                               const void* dO, const float* L, float* dQ, float* D, float c,
                               float s, int T, int Hq, int Hkv, void* stream) {
  const int st = sattn_bwd_query_check(Q, K, Vt, O, dO, L, dQ, D, c, s, T, Hq, Hkv);
  if (st != SATTN_OK) return st;
  const int dst = check_device();
  if (dst != SATTN_OK) return dst;
  launch_query(static_cast<const half_t*>(Q), static_cast<const half_t*>(K),
               static_cast<const half_t*>(Vt), static_cast<const half_t*>(O),
               static_cast<const half_t*>(dO), L, dQ, D, c, s, T, Hq, Hkv,
               static_cast<hipStream_t>(stream));
  return hipGetLastError() == hipSuccess ? SATTN_OK : SATTN_ERR_LAUNCH;
}

extern "C" int sattn_bwd_key(const void* Q, const void* K, const void* Vt, const void* dO,
                             const float* L, const float* D, float* dK, float* dVt,
                             void* workspace, unsigned long long workspace_bytes, float c,
                             float s, int T, int Hq, int Hkv, void* stream) {
  const int st = sattn_bwd_key_check(Q, K, Vt, dO, L, D, dK, dVt, workspace, workspace_bytes, c,
                                     s, T, Hq, Hkv);
  if (st != SATTN_OK) return st;
  const int dst = check_device();
  if (dst != SATTN_OK) return dst;
  launch_key(static_cast<const half_t*>(Q), static_cast<const half_t*>(K),
             static_cast<const half_t*>(Vt), static_cast<const half_t*>(dO), L, D, dK, dVt,
             workspace, c, s, T, Hq, Hkv, static_cast<hipStream_t>(stream));
  return hipGetLastError() == hipSuccess ? SATTN_OK : SATTN_ERR_LAUNCH;
}

extern "C" int sattn_bwd(const void* Q, const void* K, const void* Vt, const void* O,
                         const void* dO, const float* L, float* dQ, float* dK, float* dVt,
                         float* D, void* workspace, unsigned long long workspace_bytes, float c,
                         float s, int T, int Hq, int Hkv, void* stream) {
  const int st = sattn_bwd_check(Q, K, Vt, O, dO, L, dQ, dK, dVt, D, workspace, workspace_bytes,
                                 c, s, T, Hq, Hkv);
  if (st != SATTN_OK) return st;
  const int dst = check_device();
  if (dst != SATTN_OK) return dst;
  const hipStream_t strm = static_cast<hipStream_t>(stream);
  const half_t* q = static_cast<const half_t*>(Q);
  const half_t* k = static_cast<const half_t*>(K);
  const half_t* v = static_cast<const half_t*>(Vt);
  const half_t* g = static_cast<const half_t*>(dO);
  launch_query(q, k, v, static_cast<const half_t*>(O), g, L, dQ, D, c, s, T, Hq, Hkv, strm);
  launch_key(q, k, v, g, L, D, dK, dVt, workspace, c, s, T, Hq, Hkv, strm);
  return hipGetLastError() == hipSuccess ? SATTN_OK : SATTN_ERR_LAUNCH;
}
