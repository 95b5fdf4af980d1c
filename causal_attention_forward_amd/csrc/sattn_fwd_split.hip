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
// token-major) and m + log2 l.  Here every tile moves the maximum, as the
// page's tile body does.
//
// gfx950 design:
//  * Workgroup = four waves on one 32-row query block of one head; wave w
//    takes key tiles w, w + 4, w + 8, ... up to the block's diagonal, so a
//    block's key range is walked four times faster than by one wave.
//  * No LDS staging and no barrier in the loop: a wave reads its K rows and
//    V^T rows straight from global memory (L2) as 16-byte operand loads, the
//    next tile's loads in flight while the current tile is computed.  Given V
//    as rows, the V^T operand is gathered with 2-byte loads (lanes of a load
//    hold consecutive d, so each load still reads whole row segments).
//  * S^T = K Q^T and O^T = V^T P^T on v_mfma_f32_32x32x16_f16 (a lane owns one
//    query and 16 keys, so a row's max and sum are in-lane plus one exchange
//    with the lane 32 away); K rows are permuted so each lane's 8 keys per
//    16-key slice of P^T are consecutive (one 16-byte V^T read per operand).
//  * The merge: waves 1..3 leave m, l and O^T in LDS; wave 0 forms
//    M = max m_w, l = sum l_w 2^(m_w - M), O = sum O_w 2^(m_w - M) and writes
//    O / l and M + log2 l.
#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>

#include "sattn.h"
#include "sattn_internal.h"

namespace {

typedef _Float16 half_t;
typedef _Float16 half4 __attribute__((ext_vector_type(4)));
typedef _Float16 half8 __attribute__((ext_vector_type(8)));
typedef float float4v __attribute__((ext_vector_type(4)));
typedef float float16v __attribute__((ext_vector_type(16)));

constexpr int kD = SATTN_HEAD_DIM;
constexpr int kWaves = 4;
constexpr int kXcds = 8;

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

struct Tile {
  half8 k[8];  // K operand: key rows krow(n) (+32), d = 16 kk + 8g ..    (index 2 kk + half)
  half8 v[8];  // V^T operand: d rows n (+32), keys 16 ks + 8g ..          (index 2 ks + half)
};

template <bool VT_VEC, bool VROWS>
__global__ void __launch_bounds__(64 * kWaves, 2)
sattn_fwd_split_kernel(const half_t* __restrict__ Q, const half_t* __restrict__ K,
                       const half_t* __restrict__ Vt, half_t* __restrict__ O,
                       float* __restrict__ L, float c, int T, int Hq, int G, int nBlocks) {
  __shared__ float xo[kWaves - 1][2][16][64];  // waves 1..3: O^T accumulators, lane-major
  __shared__ float xm[kWaves - 1][64], xl[kWaves - 1][64];

  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lane = tid & 63;
  const int n = lane & 31;
  const int g = lane >> 5;

  // XCD-contiguous order: K/V head first, query blocks heaviest first, then
  // the group's query heads
  const int nWg = gridDim.x, b = blockIdx.x;
  const int lid = (b % kXcds) * (nWg / kXcds) + min(b % kXcds, nWg % kXcds) + b / kXcds;
  const int kv = lid / (nBlocks * G);
  const int rem = lid - kv * nBlocks * G;
  const int blk = nBlocks - 1 - rem / G;
  const int h = kv * G + rem % G;

  const int row = 32 * blk + n;
  const int need = min(T - 1, 32 * blk + 31) / 64 + 1;  // key tiles up to the diagonal

  half8 qf[4];
#pragma unroll
  for (int kk = 0; kk < 4; ++kk)
    qf[kk] = row < T ? ld8(Q + ((size_t)h * T + row) * kD + 16 * kk + 8 * g) : half8{};

  const half_t* Kh = K + (size_t)kv * T * kD;
  const half_t* Vh = Vt + (size_t)kv * kD * T;
  auto load = [&](int kt, Tile& t) {
    const int key0 = kt * 64;
#pragma unroll
    for (int kk = 0; kk < 4; ++kk)
#pragma unroll
      for (int hf = 0; hf < 2; ++hf) {
        const int key = key0 + 32 * hf + krow(n);
        t.k[2 * kk + hf] = key < T ? ld8(Kh + (size_t)key * kD + 16 * kk + 8 * g) : half8{};
      }
#pragma unroll
    for (int ks = 0; ks < 4; ++ks)
#pragma unroll
      for (int hf = 0; hf < 2; ++hf) {
        const int d = 32 * hf + n, k0 = key0 + 16 * ks + 8 * g;
        const half_t* src = Vh + (size_t)d * T + k0;
        if (VROWS) {  // V rows [T][64]: element (key, d) at key * 64 + d
          half8 x;
#pragma unroll
          for (int e = 0; e < 8; ++e) x[e] = k0 + e < T ? Vh[(size_t)(k0 + e) * kD + d] : (half_t)0;
          t.v[2 * ks + hf] = x;
        } else if (VT_VEC && k0 + 7 < T) {
          t.v[2 * ks + hf] = ld8(src);
        } else {
          half8 x;
#pragma unroll
          for (int e = 0; e < 8; ++e) x[e] = k0 + e < T ? src[e] : (half_t)0;
          t.v[2 * ks + hf] = x;
        }
      }
  };

  float m = -INFINITY, l = 0.0f;
  float16v o0 = {}, o1 = {};
  const int swapAddr = (lane ^ 32) << 2;
  Tile cur, nxt;
  int kt = wave;
  if (kt < need) load(kt, cur);
  while (kt < need) {
    const int kn = kt + kWaves;
    if (kn < need) load(kn, nxt);
    float16v s0 = {}, s1 = {};
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) {
      s0 = mfma(cur.k[2 * kk], qf[kk], s0);
      s1 = mfma(cur.k[2 * kk + 1], qf[kk], s1);
    }
    if (kt == need - 1) {  // the tile crossing the block's diagonal
      const int lim = row - kt * 64 - 8 * g;
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const int k = 16 * (i >> 3) + (i & 7);
        if (k > lim) s0[i] = -INFINITY;
        if (k + 32 > lim) s1[i] = -INFINITY;
      }
    }
    float x = -INFINITY;
#pragma unroll
    for (int i = 0; i < 16; ++i) x = fmaxf(x, fmaxf(s0[i], s1[i]));
    x = fmaxf(x, xlane(x, swapAddr));
    const float m_new = fmaxf(m, x * c);  // finite: key 64 kt <= row for every row
    const float alpha = __builtin_amdgcn_exp2f(m - m_new);
    m = m_new;
    float lsum = 0.0f;
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      s0[i] = __builtin_amdgcn_exp2f(fmaf(s0[i], c, -m));
      s1[i] = __builtin_amdgcn_exp2f(fmaf(s1[i], c, -m));
      lsum += s0[i] + s1[i];
    }
    l = l * alpha + lsum;
    o0 *= alpha;
    o1 *= alpha;
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
      o0 = mfma(cur.v[2 * ks], p[ks], o0);
      o1 = mfma(cur.v[2 * ks + 1], p[ks], o1);
    }
    if (kn < need) cur = nxt;
    kt = kn;
  }

  // merge the four waves' (m, l, O) of the same 32 rows; l is a partial sum
  // per lane (keys of its half), so the pair's sums are added first
  l += xlane(l, swapAddr);
  if (wave > 0) {
    const int w = wave - 1;
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      xo[w][0][i][lane] = o0[i];
      xo[w][1][i][lane] = o1[i];
    }
    xm[w][lane] = m;
    xl[w][lane] = l;
  }
  __syncthreads();
  if (wave != 0) return;
  float M = m;
#pragma unroll
  for (int w = 0; w < kWaves - 1; ++w) M = fmaxf(M, xm[w][lane]);
  const float a0 = __builtin_amdgcn_exp2f(m - M);
  float lt = l * a0;
  o0 *= a0;
  o1 *= a0;
#pragma unroll
  for (int w = 0; w < kWaves - 1; ++w) {
    const float aw = __builtin_amdgcn_exp2f(xm[w][lane] - M);  // 0 for a wave with no tile
    lt += xl[w][lane] * aw;
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      o0[i] += xo[w][0][i][lane] * aw;
      o1[i] += xo[w][1][i][lane] * aw;
    }
  }
  if (row < T) {
    const float inv = __builtin_amdgcn_rcpf(lt);
    half_t* orow = O + (size_t)row * Hq * kD + (size_t)h * kD + 4 * g;
#pragma unroll
    for (int q4 = 0; q4 < 4; ++q4) {
      const float4v va = {o0[4 * q4], o0[4 * q4 + 1], o0[4 * q4 + 2], o0[4 * q4 + 3]};
      const float4v vb = {o1[4 * q4], o1[4 * q4 + 1], o1[4 * q4 + 2], o1[4 * q4 + 3]};
      *reinterpret_cast<half4*>(orow + 8 * q4) = __builtin_convertvector(va * inv, half4);
      *reinterpret_cast<half4*>(orow + 32 + 8 * q4) = __builtin_convertvector(vb * inv, half4);
    }
    if (g == 0) L[(size_t)h * T + row] = M + __builtin_amdgcn_logf(lt);
  }
}

}  // namespace

void sattn_fwd_split_launch(const void* Q, const void* K, const void* Vt, void* O, float* L,
                            float c, int T, int Hq, int Hkv, bool vrows, hipStream_t stream) {
  const int G = Hq / Hkv;
  const int nBlocks = (T + 31) / 32;
  const dim3 grid((unsigned)nBlocks * (unsigned)Hq);
  const half_t* q = static_cast<const half_t*>(Q);
  const half_t* k = static_cast<const half_t*>(K);
  const half_t* v = static_cast<const half_t*>(Vt);
  half_t* o = static_cast<half_t*>(O);
  if (vrows)
    hipLaunchKernelGGL((sattn_fwd_split_kernel<false, true>), grid, dim3(64 * kWaves), 0, stream,
                       q, k, v, o, L, c, T, Hq, G, nBlocks);
  else if (T % 8 == 0)
    hipLaunchKernelGGL((sattn_fwd_split_kernel<true, false>), grid, dim3(64 * kWaves), 0, stream,
                       q, k, v, o, L, c, T, Hq, G, nBlocks);
  else
    hipLaunchKernelGGL((sattn_fwd_split_kernel<false, false>), grid, dim3(64 * kWaves), 0, stream,
                       q, k, v, o, L, c, T, Hq, G, nBlocks);
}
