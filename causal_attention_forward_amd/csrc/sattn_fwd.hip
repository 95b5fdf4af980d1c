// The causal streaming-attention forward for gfx950 (CDNA4), and its C entry.
//
// Method (StreamingAttentionSM86 page, header comment and tile body of the
// forward realization): for each 64-key tile up to the diagonal, scores are
// formed on the matrix cores, scaled to base-2 units t = S*c, folded into a
// running row maximum m, row sum l and weighted sum O by the merge rule for
// normalised weighted sums (a new maximum m' scales the old l and O by
// 2^(m - m')), and the tile's P V is added with P = 2^(t - m') rounded to
// binary16.  The epilogue writes O / l (binary16, token-major) and
// m + log2 l (binary32).
//
// gfx950 design (not the page's SM86 one):
//  * The transposed problem is computed: S^T = K Q^T and O^T = V^T P^T on
//    v_mfma_f32_32x32x16_f16.  In the 32x32 accumulator layout a lane holds
//    one column (one query) and 16 rows (keys), so a row's max and sum are
//    in-lane except for one exchange with the lane 32 away, and the S^T
//    accumulator already is the P^T operand of the second product: no LDS
//    round trip and no cross-lane shuffle for P.
//  * A workgroup is four wave64s.  Each wave owns 32 query rows of one query
//    head; the workgroup's waves are GW query heads of one GQA group times
//    4/GW row blocks, so one K/V tile in LDS feeds 128 query rows.
//  * K and V^T tiles (64 keys) are staged through LDS, double-buffered, with
//    a 16-byte-chunk XOR swizzle; the next tile's global loads are in flight
//    while the current one is computed.
//  * Tiles past the causal diagonal are never visited; waves whose rows end
//    before a tile skip its arithmetic; only tiles that cross the diagonal
//    are masked.  Loads past T are zero-filled and rows past T are not
//    stored, so T need not be a multiple of 64.
//  * The launch is a 1-D grid ordered heaviest row tile first.
#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>
#include <string.h>

#include <atomic>

#include "sattn.h"

namespace {

typedef _Float16 half_t;
typedef _Float16 half4 __attribute__((ext_vector_type(4)));
typedef _Float16 half8 __attribute__((ext_vector_type(8)));
typedef float float4v __attribute__((ext_vector_type(4)));
typedef float float8v __attribute__((ext_vector_type(8)));
typedef float float16v __attribute__((ext_vector_type(16)));
typedef unsigned int uint4v __attribute__((ext_vector_type(4)));

constexpr int kD = SATTN_HEAD_DIM;  // head width
constexpr int kBN = 64;             // keys per tile
constexpr int kWaves = 4;
constexpr int kThreads = 64 * kWaves;
constexpr int kTileHalfs = kBN * kD;  // one K or V^T tile: 64 x 64 binary16

// 16-byte chunk c of LDS row r is stored at chunk c ^ (r & 7).
__device__ __forceinline__ int lds_index(int r, int chunk) { return r * 64 + ((chunk ^ (r & 7)) << 3); }

__device__ __forceinline__ half8 to_half8(float8v x) { return __builtin_convertvector(x, half8); }

template <int GW, bool VT_VEC>
__global__ void __launch_bounds__(kThreads)
sattn_fwd_kernel(const half_t* __restrict__ Q, const half_t* __restrict__ K,
                 const half_t* __restrict__ Vt, half_t* __restrict__ O, float* __restrict__ L,
                 float c, int T, int Hq, int Hkv, int G, int nRowTiles, int nHeadGroups) {
  constexpr int BM = 32 * (kWaves / GW);  // query rows per workgroup
  __shared__ __attribute__((aligned(16))) half_t sK[2][kTileHalfs];
  __shared__ __attribute__((aligned(16))) half_t sV[2][kTileHalfs];

  const int tid = threadIdx.x;
  const int wave = tid >> 6;
  const int lane = tid & 63;
  const int n = lane & 31;  // accumulator column: the query within the wave; A-operand row
  const int g = lane >> 5;  // which half of the k range / row octets this lane holds

  const int perTile = Hkv * nHeadGroups;
  const int tileOrd = blockIdx.x / perTile;
  const int rest = blockIdx.x - tileOrd * perTile;
  const int rt = nRowTiles - 1 - tileOrd;  // heaviest row tile first
  const int kv = rest / nHeadGroups;
  const int hg = rest - kv * nHeadGroups;
  const int h = kv * G + hg * GW + (wave % GW);
  const int r0 = rt * BM + (wave / GW) * 32;  // this wave's first query row
  const int row = r0 + n;                     // this lane's query row
  const int wgLast = min(T - 1, rt * BM + BM - 1);
  const int nkt = wgLast / kBN + 1;  // key tiles 0 .. the diagonal one

  // Q^T as the B operand of S^T = K Q^T: lane (n, g) holds Q[row][16kk + 8g .. +8].
  half8 qf[4];
  {
    const half_t* qrow = Q + ((size_t)h * T + row) * kD;
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) {
      if (row < T)
        qf[kk] = *reinterpret_cast<const half8*>(qrow + 16 * kk + 8 * g);
      else
        qf[kk] = half8{};
    }
  }

  // Global -> register staging of one K and one V^T tile: 2 x 512 chunks of
  // 16 bytes, four per thread.
  uint4v stK[2], stV[2];
  const half_t* Kh = K + (size_t)kv * T * kD;
  const half_t* Vh = Vt + (size_t)kv * kD * T;
  auto load_tile = [&](int kt) {
    const int key0 = kt * kBN;
#pragma unroll
    for (int p = 0; p < 2; ++p) {
      const int cidx = tid + p * kThreads;
      const int r = cidx >> 3, ch = cidx & 7;
      const int key = key0 + r;
      stK[p] = key < T ? *reinterpret_cast<const uint4v*>(Kh + (size_t)key * kD + ch * 8) : uint4v{};
      const half_t* vrow = Vh + (size_t)r * T;  // V^T row d = r
      const int k8 = key0 + ch * 8;
      if (VT_VEC) {
        stV[p] = k8 < T ? *reinterpret_cast<const uint4v*>(vrow + k8) : uint4v{};
      } else {
        half8 v;
#pragma unroll
        for (int e = 0; e < 8; ++e) v[e] = (k8 + e < T) ? vrow[k8 + e] : (half_t)0;
        stV[p] = __builtin_bit_cast(uint4v, v);
      }
    }
  };
  auto store_tile = [&](int buf) {
#pragma unroll
    for (int p = 0; p < 2; ++p) {
      const int cidx = tid + p * kThreads;
      const int r = cidx >> 3, ch = cidx & 7;
      *reinterpret_cast<uint4v*>(&sK[buf][lds_index(r, ch)]) = stK[p];
      *reinterpret_cast<uint4v*>(&sV[buf][lds_index(r, ch)]) = stV[p];
    }
  };

  float m = -INFINITY;  // running row maximum of t (base 2), shared by lanes n and n+32
  float l = 0.0f;       // this lane's partial row sum of P
  float16v o0 = {}, o1 = {};  // O^T accumulators: d rows 0..31 and 32..63, column = query

  load_tile(0);
  store_tile(0);
  for (int kt = 0; kt < nkt; ++kt) {
    const int buf = kt & 1;
    if (kt + 1 < nkt) load_tile(kt + 1);
    __syncthreads();
    const int key0 = kt * kBN;
    if (key0 <= r0 + 31) {  // otherwise every key of the tile is after every row of the wave
      const half_t* ks = sK[buf];
      const half_t* vs = sV[buf];

      // S^T (keys x queries): s0 holds keys key0 + 0..31, s1 keys key0 + 32..63.
      float16v s0 = {}, s1 = {};
#pragma unroll
      for (int kk = 0; kk < 4; ++kk) {
        const half8 a0 = *reinterpret_cast<const half8*>(&ks[lds_index(n, 2 * kk + g)]);
        const half8 a1 = *reinterpret_cast<const half8*>(&ks[lds_index(32 + n, 2 * kk + g)]);
        s0 = __builtin_amdgcn_mfma_f32_32x32x16_f16(a0, qf[kk], s0, 0, 0, 0);
        s1 = __builtin_amdgcn_mfma_f32_32x32x16_f16(a1, qf[kk], s1, 0, 0, 0);
      }

      // Causal mask: accumulator element i of lane (n, g) is key
      // key0 + 8*(i/4) + 4g + i%4 (+32 in s1); it is masked when it exceeds the row.
      if (key0 + kBN - 1 > r0) {
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const int key = key0 + 8 * (i >> 2) + 4 * g + (i & 3);
          if (key > row) s0[i] = -INFINITY;
          if (key + 32 > row) s1[i] = -INFINITY;
        }
      }

      // The row maximum over the tile's 64 keys (raw scores; c > 0 keeps the order).
      float mx = fmaxf(s0[0], s1[0]);
#pragma unroll
      for (int i = 1; i < 16; ++i) mx = fmaxf(mx, fmaxf(s0[i], s1[i]));
      mx = fmaxf(mx, __shfl_xor(mx, 32));
      const float m_new = fmaxf(m, mx * c);
      const float alpha = __builtin_amdgcn_exp2f(m - m_new);  // 0 on the first tile
      const float neg_m = -m_new;
      m = m_new;

      // P = 2^(S c - m'), its unrounded row sum, then the rescale of l and O.
      float ls = 0.0f;
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        s0[i] = __builtin_amdgcn_exp2f(fmaf(s0[i], c, neg_m));
        s1[i] = __builtin_amdgcn_exp2f(fmaf(s1[i], c, neg_m));
        ls += s0[i] + s1[i];
      }
      l = l * alpha + ls;
      o0 *= alpha;
      o1 *= alpha;

      // P^T as the B operand of O^T = V^T P^T: slice ks covers accumulator
      // elements 8*(ks%2) .. +7 of s(ks/2), i.e. keys 16ks + 8*(j/4) + 4g + j%4.
      const half8 p0 = to_half8(__builtin_shufflevector(s0, s0, 0, 1, 2, 3, 4, 5, 6, 7));
      const half8 p1 = to_half8(__builtin_shufflevector(s0, s0, 8, 9, 10, 11, 12, 13, 14, 15));
      const half8 p2 = to_half8(__builtin_shufflevector(s1, s1, 0, 1, 2, 3, 4, 5, 6, 7));
      const half8 p3 = to_half8(__builtin_shufflevector(s1, s1, 8, 9, 10, 11, 12, 13, 14, 15));
      const half8 pb[4] = {p0, p1, p2, p3};

      // V^T as the A operand, matching that key order: lane (n, g) reads
      // d row (32dt + n), keys 16ks + 4g .. +3 and 16ks + 8 + 4g .. +3.
#pragma unroll
      for (int ks4 = 0; ks4 < 4; ++ks4) {
#pragma unroll
        for (int dt = 0; dt < 2; ++dt) {
          const int d = 32 * dt + n;
          const half4 lo = *reinterpret_cast<const half4*>(&vs[lds_index(d, 2 * ks4) + 4 * g]);
          const half4 hi = *reinterpret_cast<const half4*>(&vs[lds_index(d, 2 * ks4 + 1) + 4 * g]);
          const half8 a = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
          if (dt == 0)
            o0 = __builtin_amdgcn_mfma_f32_32x32x16_f16(a, pb[ks4], o0, 0, 0, 0);
          else
            o1 = __builtin_amdgcn_mfma_f32_32x32x16_f16(a, pb[ks4], o1, 0, 0, 0);
        }
      }
    }
    if (kt + 1 < nkt) store_tile(buf ^ 1);
  }

  // Epilogue: the row sum over both lane halves, O / l, and m + log2 l.
  const float lt = l + __shfl_xor(l, 32);
  const float inv = __builtin_amdgcn_rcpf(lt);
  const float lse = m + __builtin_amdgcn_logf(lt);
  if (row < T) {
    half_t* orow = O + (size_t)row * Hq * kD + (size_t)h * kD;
#pragma unroll
    for (int q4 = 0; q4 < 4; ++q4) {
      // accumulator elements 4q4 .. 4q4+3 are d = 8q4 + 4g + 0..3 (+32 in o1)
      const float4v a = {o0[4 * q4], o0[4 * q4 + 1], o0[4 * q4 + 2], o0[4 * q4 + 3]};
      const float4v b = {o1[4 * q4], o1[4 * q4 + 1], o1[4 * q4 + 2], o1[4 * q4 + 3]};
      *reinterpret_cast<half4*>(orow + 8 * q4 + 4 * g) = __builtin_convertvector(a * inv, half4);
      *reinterpret_cast<half4*>(orow + 32 + 8 * q4 + 4 * g) = __builtin_convertvector(b * inv, half4);
    }
    if (g == 0) L[(size_t)h * T + row] = lse;
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

template <int GW, bool VT_VEC>
void launch(const half_t* Q, const half_t* K, const half_t* Vt, half_t* O, float* L, float c,
            int T, int Hq, int Hkv, hipStream_t stream) {
  constexpr int BM = 32 * (kWaves / GW);
  const int G = Hq / Hkv;
  const int nRowTiles = (T + BM - 1) / BM;
  const int nHeadGroups = G / GW;
  const unsigned grid = (unsigned)nRowTiles * (unsigned)Hkv * (unsigned)nHeadGroups;
  hipLaunchKernelGGL((sattn_fwd_kernel<GW, VT_VEC>), dim3(grid), dim3(kThreads), 0, stream, Q, K,
                     Vt, O, L, c, T, Hq, Hkv, G, nRowTiles, nHeadGroups);
}

template <int GW>
void launch_gw(const half_t* Q, const half_t* K, const half_t* Vt, half_t* O, float* L, float c,
               int T, int Hq, int Hkv, hipStream_t stream) {
  if (T % 8 == 0)
    launch<GW, true>(Q, K, Vt, O, L, c, T, Hq, Hkv, stream);
  else
    launch<GW, false>(Q, K, Vt, O, L, c, T, Hq, Hkv, stream);
}

}  // namespace

extern "C" int sattn_fwd(const void* Q, const void* K, const void* Vt, void* O, float* L,
                         float c, int T, int Hq, int Hkv, void* stream) {
  const int st = sattn_fwd_check(Q, K, Vt, O, L, c, T, Hq, Hkv);
  if (st != SATTN_OK) return st;
  const int dst = check_device();
  if (dst != SATTN_OK) return dst;
  const half_t* q = static_cast<const half_t*>(Q);
  const half_t* k = static_cast<const half_t*>(K);
  const half_t* v = static_cast<const half_t*>(Vt);
  half_t* o = static_cast<half_t*>(O);
  hipStream_t s = static_cast<hipStream_t>(stream);
  const int G = Hq / Hkv;
  if (G % 4 == 0)
    launch_gw<4>(q, k, v, o, L, c, T, Hq, Hkv, s);
  else if (G % 2 == 0)
    launch_gw<2>(q, k, v, o, L, c, T, Hq, Hkv, s);
  else
    launch_gw<1>(q, k, v, o, L, c, T, Hq, Hkv, s);
  return hipGetLastError() == hipSuccess ? SATTN_OK : SATTN_ERR_LAUNCH;
}
