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
//  * A workgroup is four wave64s.  Each wave owns 32 query rows of one query
//    head; the workgroup's waves are GW query heads of one GQA group times
//    4/GW row blocks, so one K/V tile in LDS feeds 128 query rows.
//  * K and V^T tiles (64 keys) are staged through LDS, double-buffered, rows
//    padded to 144 bytes so the 16-byte operand reads of 16 lanes hit 64
//    distinct banks.  The next tile's global loads are in flight while the
//    current one is computed.  K is read through a buffer descriptor whose
//    range ends at T, so rows past T arrive as zeros.
//  * The reference maximum is moved lazily: l and O are rescaled only when
//    some row's tile maximum exceeds its reference by more than kLazy (base-2
//    units).  The merge rule holds for any reference, so this changes only
//    rounding, and P stays below 2^kLazy (far inside binary16).
//  * Tiles past the causal diagonal are never visited, waves whose rows end
//    before a tile skip its arithmetic, and only tiles that cross the
//    diagonal are masked.  Rows past T are computed on zero queries and not
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
typedef int int4v __attribute__((ext_vector_type(4)));

constexpr int kD = SATTN_HEAD_DIM;  // head width
constexpr int kBN = 64;             // keys per tile
constexpr int kWaves = 4;
constexpr int kThreads = 64 * kWaves;
constexpr int kRowHalfs = kD + 8;                // LDS row: 64 values + 16 bytes of padding
constexpr int kTileHalfs = kBN * kRowHalfs;      // one K or V^T tile in LDS
constexpr float kLazy = 8.0f;                    // rescale threshold, base-2 units
constexpr int kBufferWord3 = 0x00020000;         // raw buffer, 32-bit data format

__device__ __forceinline__ half8 to_half8(float8v x) { return __builtin_convertvector(x, half8); }

__device__ __forceinline__ float16v mfma(half8 a, half8 b, float16v c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b, c, 0, 0, 0);
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

template <int GW, bool VT_VEC>
__global__ void __launch_bounds__(kThreads, 2)
sattn_fwd_kernel(const half_t* __restrict__ Q, const half_t* __restrict__ K,
                 const half_t* __restrict__ Vt, half_t* __restrict__ O, float* __restrict__ L,
                 float c, int T, int Hq, int Hkv, int G, int nRowTiles, int nHeadGroups) {
  constexpr int BM = 32 * (kWaves / GW);  // query rows per workgroup
  __shared__ __attribute__((aligned(16))) half_t smem[4 * kTileHalfs];  // K0 V0 K1 V1

  const int tid = threadIdx.x;
  const int wave = tid >> 6;
  const int lane = tid & 63;
  const int n = lane & 31;  // accumulator column (query) / operand row
  const int g = lane >> 5;  // operand k-half / accumulator row octet

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
    const half_t* qrow = Q + ((size_t)h * T + row) * kD + 8 * g;
#pragma unroll
    for (int kk = 0; kk < 4; ++kk)
      qf[kk] = row < T ? *reinterpret_cast<const half8*>(qrow + 16 * kk) : half8{};
  }

  // Global -> register staging of one tile: 512 K chunks and 512 V^T chunks
  // of 16 bytes; thread t owns chunks t and t + 256 of each.
  const __amdgpu_buffer_rsrc_t krsrc = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<half_t*>(K + (size_t)kv * T * kD), 0, T * kD * 2, kBufferWord3);
  const half_t* Vh = Vt + (size_t)kv * kD * T;
  const int cr = tid >> 3, cc = tid & 7;  // chunk p: row cr + 32p, column chunk cc
  int4v stK[2], stV[2];
  auto load_tile = [&](int kt) {
    const int key0 = kt * kBN;
#pragma unroll
    for (int p = 0; p < 2; ++p) {
      const int r = cr + 32 * p;
      stK[p] = __builtin_amdgcn_raw_buffer_load_b128(krsrc, ((key0 + r) * kD + cc * 8) * 2, 0, 0);
      const half_t* vsrc = Vh + (size_t)r * T + key0 + cc * 8;  // V^T row d = r
      if (VT_VEC && key0 + kBN <= T) {  // whole tile inside T (uniform)
        stV[p] = *reinterpret_cast<const int4v*>(vsrc);
      } else if (VT_VEC) {  // T % 8 == 0: a chunk is wholly inside or outside
        stV[p] = key0 + cc * 8 < T ? *reinterpret_cast<const int4v*>(vsrc) : int4v{};
      } else {
        half8 v;
#pragma unroll
        for (int e = 0; e < 8; ++e) v[e] = (key0 + cc * 8 + e < T) ? vsrc[e] : (half_t)0;
        stV[p] = __builtin_bit_cast(int4v, v);
      }
    }
  };
  auto store_tile = [&](int buf) {
    half_t* ks = smem + buf * 2 * kTileHalfs;
#pragma unroll
    for (int p = 0; p < 2; ++p) {
      const int off = (cr + 32 * p) * kRowHalfs + cc * 8;
      *reinterpret_cast<int4v*>(ks + off) = stK[p];
      *reinterpret_cast<int4v*>(ks + kTileHalfs + off) = stV[p];
    }
  };

  const int swapAddr = (lane ^ 32) << 2;  // byte address of the lane 32 away

  // Per-lane LDS operand offsets (halfs) within a tile.
  const int kOff = krow(n) * kRowHalfs + 8 * g;  // + 32s rows, + 16kk columns
  const int vOff = n * kRowHalfs + 8 * g;        // + 32dt rows, + 16ks columns

  float m = -INFINITY;  // reference maximum of t (base 2), equal on lanes n and n+32
  float l = 0.0f;       // this lane's partial row sum of P
  float16v o0 = {}, o1 = {};  // O^T: d rows 0..31 and 32..63 of this lane's query

  load_tile(0);
  store_tile(0);
  for (int kt = 0; kt < nkt; ++kt) {
    const int buf = kt & 1;
    if (kt + 1 < nkt) load_tile(kt + 1);
    __syncthreads();
    const int key0 = kt * kBN;
    if (key0 <= r0 + 31) {  // otherwise every key of the tile is after every row of the wave
      const half_t* ks = smem + buf * 2 * kTileHalfs;
      const half_t* vs = ks + kTileHalfs;

      // S^T (keys x queries): element i of s0 is key key0 + 16*(i/8) + 8g + i%8; s1 is +32.
      float16v s0, s1;
      {
        const half8 a0 = *reinterpret_cast<const half8*>(ks + kOff);
        const half8 a1 = *reinterpret_cast<const half8*>(ks + kOff + 32 * kRowHalfs);
        s0 = mfma(a0, qf[0], float16v{});
        s1 = mfma(a1, qf[0], float16v{});
      }
#pragma unroll
      for (int kk = 1; kk < 4; ++kk) {
        const half8 a0 = *reinterpret_cast<const half8*>(ks + kOff + 16 * kk);
        const half8 a1 = *reinterpret_cast<const half8*>(ks + kOff + 32 * kRowHalfs + 16 * kk);
        s0 = mfma(a0, qf[kk], s0);
        s1 = mfma(a1, qf[kk], s1);
      }

      // Causal mask on tiles that reach past the wave's first row.
      if (key0 + kBN - 1 > r0) {
        const int lim = row - key0 - 8 * g;  // element i is masked when 16*(i/8) + i%8 (+32) > lim
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const int k = 16 * (i >> 3) + (i & 7);
          if (k > lim) s0[i] = -INFINITY;
          if (k + 32 > lim) s1[i] = -INFINITY;
        }
      }

      // The tile's row maximum (raw scores; c > 0 keeps the order), both lane halves.
      float mx = __builtin_fmaxf(s0[0], s1[0]);
#pragma unroll
      for (int i = 1; i < 16; ++i) mx = __builtin_fmaxf(mx, __builtin_fmaxf(s0[i], s1[i]));
      mx = __builtin_fmaxf(mx, xlane(mx, swapAddr)) * c;

      // Move the reference only when some row of the wave outgrew it by kLazy.
      if (__builtin_amdgcn_ballot_w64(mx > m + kLazy) != 0) {
        const float m_new = __builtin_fmaxf(m, mx);
        const float alpha = __builtin_amdgcn_exp2f(m - m_new);  // 0 on a row's first tile
        m = m_new;
        l *= alpha;
        o0 *= alpha;
        o1 *= alpha;
      }

      // P = 2^(S c - m) and its unrounded row sum.
      const float neg_m = -m;
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        s0[i] = __builtin_amdgcn_exp2f(__builtin_fmaf(s0[i], c, neg_m));
        s1[i] = __builtin_amdgcn_exp2f(__builtin_fmaf(s1[i], c, neg_m));
      }
      float ls0 = s0[0], ls1 = s1[0];
#pragma unroll
      for (int i = 1; i < 16; ++i) {
        ls0 += s0[i];
        ls1 += s1[i];
      }
      l += ls0 + ls1;

      // O^T += V^T P^T over four 16-key slices: slice ks takes elements
      // 8*(ks%2) .. +7 of s(ks/2), i.e. keys 16ks + 8g .. +7, as its B operand.
      const half8 p0 = to_half8(__builtin_shufflevector(s0, s0, 0, 1, 2, 3, 4, 5, 6, 7));
      const half8 p1 = to_half8(__builtin_shufflevector(s0, s0, 8, 9, 10, 11, 12, 13, 14, 15));
      const half8 p2 = to_half8(__builtin_shufflevector(s1, s1, 0, 1, 2, 3, 4, 5, 6, 7));
      const half8 p3 = to_half8(__builtin_shufflevector(s1, s1, 8, 9, 10, 11, 12, 13, 14, 15));
      const half8 pb[4] = {p0, p1, p2, p3};
#pragma unroll
      for (int ks4 = 0; ks4 < 4; ++ks4) {
        const half8 v0 = *reinterpret_cast<const half8*>(vs + vOff + 16 * ks4);
        const half8 v1 = *reinterpret_cast<const half8*>(vs + vOff + 32 * kRowHalfs + 16 * ks4);
        o0 = mfma(v0, pb[ks4], o0);
        o1 = mfma(v1, pb[ks4], o1);
      }
    }
    if (kt + 1 < nkt) store_tile(buf ^ 1);
  }

  // Epilogue: the row sum over both lane halves, O / l, and m + log2 l.
  const float lt = l + xlane(l, swapAddr);
  const float inv = __builtin_amdgcn_rcpf(lt);
  const float lse = m + __builtin_amdgcn_logf(lt);
  if (row < T) {
    half_t* orow = O + (size_t)row * Hq * kD + (size_t)h * kD + 4 * g;
#pragma unroll
    for (int q4 = 0; q4 < 4; ++q4) {
      // accumulator elements 4q4 .. 4q4+3 are d = 8q4 + 4g + 0..3 (+32 in o1)
      const float4v a = {o0[4 * q4], o0[4 * q4 + 1], o0[4 * q4 + 2], o0[4 * q4 + 3]};
      const float4v b = {o1[4 * q4], o1[4 * q4 + 1], o1[4 * q4 + 2], o1[4 * q4 + 3]};
      *reinterpret_cast<half4*>(orow + 8 * q4) = __builtin_convertvector(a * inv, half4);
      *reinterpret_cast<half4*>(orow + 32 + 8 * q4) = __builtin_convertvector(b * inv, half4);
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
