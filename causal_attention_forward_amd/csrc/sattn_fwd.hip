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
//  * Each wave is software-pipelined: while its VALUs turn the scores of tile
//    j into P, the matrix cores already form the scores of tile j+1, and the
//    P V products of tile j overlap the row sum.  K and V^T tiles (64 keys)
//    go through a ring of three LDS buffers (tile j's V^T and tile j+1's K
//    are read while tile j+2 is written), one barrier per tile; global loads
//    run one tile ahead of the ring.  LDS rows are padded to 144 bytes so the
//    16-byte operand reads of 16 lanes hit 64 distinct banks.  K is read
//    through a buffer descriptor whose range ends at T, so rows past T
//    arrive as zeros.
//  * The reference maximum is moved lazily: l and O are rescaled only when
//    some row's tile maximum exceeds its reference by more than kLazy (base-2
//    units).  The merge rule holds for any reference, so this changes only
//    rounding, and P stays below 2^kLazy (far inside binary16).
//  * Tiles past the causal diagonal are never visited, waves whose rows end
//    before a tile skip its arithmetic, and only tiles that cross the
//    diagonal are masked.  Rows past T are computed on zero queries and not
//    stored, so T need not be a multiple of 64.
//  * A workgroup takes row tiles b and n-1-b (n row tiles per head), so all
//    workgroups carry the same causal work and finish together.
#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>
#include <string.h>

#include <atomic>
#include <type_traits>

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
constexpr int kXcds = 8;                         // accelerator complex dies per MI355X

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
                 float c, int T, int Hq, int Hkv, int G, int nBlocks, int nPairs, int nSlotGroups,
                 int nHeadGroups) {
  constexpr int RS = kWaves / GW;           // row slots per workgroup
  constexpr int kBufHalfs = 2 * kTileHalfs;  // one LDS buffer: K tile, then V^T tile
  __shared__ __attribute__((aligned(16))) half_t smem[2 * kBufHalfs];

  const int tid = threadIdx.x;
  const int wave = tid >> 6;
  const int lane = tid & 63;
  const int n = lane & 31;  // accumulator column (query) / operand row
  const int g = lane >> 5;  // operand k-half / accumulator row octet

  // Query rows come in 32-row blocks; block b is paired with block
  // nBlocks-1-b, so the two together always need about nBlocks/2 + 1 key
  // tiles.  A wave owns one pair (its query tiles 0 and 1) of one head; the
  // workgroup's waves are GW heads of one GQA group times RS pairs.
  //
  // Workgroups are dealt to the eight XCDs round-robin (workgroup b runs on
  // XCD b % 8); renumbering them so that each XCD receives a contiguous run
  // of logical ids, ordered K/V head first, keeps one K/V head's tiles in
  // one XCD's L2.
  const int nWg = gridDim.x;
  const int xcd = blockIdx.x % kXcds, idx = blockIdx.x / kXcds;
  const int lid = xcd * (nWg / kXcds) + min(xcd, nWg % kXcds) + idx;
  const int perKv = nHeadGroups * nSlotGroups;
  const int kv = lid / perKv;
  const int hg = (lid - kv * perKv) / nSlotGroups;
  const int sg = lid - kv * perKv - hg * nSlotGroups;
  const int h = kv * G + hg * GW + (wave % GW);
  const int pair = sg * RS + wave / GW;
  const bool hasPair = pair < nPairs;
  const int blk0 = pair;                     // light block
  const int blk1 = nBlocks - 1 - pair;       // heavy block (== blk0 for an odd middle)
  const int rq[2] = {32 * blk0, 32 * blk1};  // first row of query tiles 0 and 1
  // key tiles each query tile needs (0 when the tile does not exist)
  const int need0 = hasPair ? min(T - 1, rq[0] + 31) / kBN + 1 : 0;
  const int need1 = (hasPair && blk1 > blk0) ? min(T - 1, rq[1] + 31) / kBN + 1 : 0;
  // key tiles the workgroup walks: the need of its first slot's heavy block,
  // the largest of its waves
  const int nkt = min(T - 1, 32 * (nBlocks - 1 - sg * RS) + 31) / kBN + 1;

  // Global -> register staging of one tile: 512 K chunks and 512 V^T chunks
  // of 16 bytes; thread t owns chunks t and t + 256 of each (rows cr, cr + 32,
  // column chunk cc).  Both planes are read through buffer descriptors: K's
  // range ends at row T, so rows past T arrive as zeros; V^T tiles wholly
  // inside T take their key offset as a scalar, and the one partial tile is
  // read with per-element guards.
  const int cr = tid >> 3, cc = tid & 7;
  const __amdgpu_buffer_rsrc_t krsrc = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<half_t*>(K + (size_t)kv * T * kD), 0, T * kD * 2, kBufferWord3);
  const half_t* Vh = Vt + (size_t)kv * kD * T;
  const __amdgpu_buffer_rsrc_t vrsrc =
      __builtin_amdgcn_make_buffer_rsrc(const_cast<half_t*>(Vh), 0, kD * T * 2, kBufferWord3);
  const int kByte = (cr * kD + cc * 8) * 2;   // + 32*128 for the second chunk, + key0*128
  const int vByte = (cr * T + cc * 8) * 2;    // + 32*T*2 for the second chunk, + key0*2
  int4v stK[2], stV[2];
  auto load_tile = [&](int kt) {
    const int key0 = kt * kBN;
#pragma unroll
    for (int p = 0; p < 2; ++p) {
      stK[p] = __builtin_amdgcn_raw_buffer_load_b128(krsrc, kByte + (key0 + 32 * p) * kD * 2, 0, 0);
      if (key0 + kBN <= T) {  // whole tile inside T (uniform)
        stV[p] = __builtin_amdgcn_raw_buffer_load_b128(vrsrc, vByte + 32 * p * T * 2, key0 * 2, 0);
      } else {
        const half_t* vsrc = Vh + (size_t)(cr + 32 * p) * T + key0 + cc * 8;  // V^T row d
        if (VT_VEC) {  // T % 8 == 0: a chunk is wholly inside or outside
          stV[p] = key0 + cc * 8 < T ? *reinterpret_cast<const int4v*>(vsrc) : int4v{};
        } else {
          half8 v;
#pragma unroll
          for (int e = 0; e < 8; ++e) v[e] = (key0 + cc * 8 + e < T) ? vsrc[e] : (half_t)0;
          stV[p] = __builtin_bit_cast(int4v, v);
        }
      }
    }
  };
  const int stOff = cr * kRowHalfs + cc * 8;  // + 32 rows for the second chunk
  auto store_tile = [&](int buf) {
    half_t* ks = smem + buf * kBufHalfs;
#pragma unroll
    for (int p = 0; p < 2; ++p) {
      *reinterpret_cast<int4v*>(ks + stOff + 32 * p * kRowHalfs) = stK[p];
      *reinterpret_cast<int4v*>(ks + kTileHalfs + stOff + 32 * p * kRowHalfs) = stV[p];
    }
  };

  const int swapAddr = (lane ^ 32) << 2;  // byte address of the lane 32 away

  // Per-lane LDS operand offsets (halfs) within a tile.
  const int kOff = krow(n) * kRowHalfs + 8 * g;  // + 32s rows, + 16kk columns
  const int vOff = n * kRowHalfs + 8 * g;        // + 32dt rows, + 16ks columns

  // Q^T as the B operand of S^T = K Q^T: lane (n, g) of query tile qt holds
  // Q[rq[qt] + n][16kk + 8g .. +8].
  half8 qf[2][4];
#pragma unroll
  for (int qt = 0; qt < 2; ++qt) {
    const int row = rq[qt] + n;
    const bool live = qt == 0 ? need0 > 0 : need1 > 0;
    const half_t* qrow = Q + ((size_t)h * T + row) * kD + 8 * g;
#pragma unroll
    for (int kk = 0; kk < 4; ++kk)
      qf[qt][kk] = (live && row < T) ? *reinterpret_cast<const half8*>(qrow + 16 * kk) : half8{};
  }

  float m[2], l[2];     // reference maximum of t (base 2) and this lane's partial row sum
  float16v o[2][2];     // O^T per query tile: d rows 0..31 and 32..63 of this lane's query
#pragma unroll
  for (int qt = 0; qt < 2; ++qt) {
    m[qt] = -INFINITY;
    l[qt] = 0.0f;
    o[qt][0] = float16v{};
    o[qt][1] = float16v{};
  }

  // Key tile j (in LDS buffer `buf`) folded into the live query tiles
  // A0, A1: every K and V^T operand read from LDS feeds each live tile.
  auto tile_body = [&](auto A0, auto A1, int j, int buf) {
    constexpr bool a0 = decltype(A0)::value, a1 = decltype(A1)::value;
    const bool act[2] = {a0, a1};
    const int key0 = j * kBN;
    const half_t* ks = smem + buf * kBufHalfs;
    const half_t* vs = ks + kTileHalfs;

    // S^T (keys x queries): element i of S[qt][sb] is key key0 + 32sb + 16*(i/8) + 8g + i%8.
    float16v S[2][2];
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) {
#pragma unroll
      for (int sb = 0; sb < 2; ++sb) {
        const half8 a = *reinterpret_cast<const half8*>(ks + kOff + 32 * sb * kRowHalfs + 16 * kk);
#pragma unroll
        for (int qt = 0; qt < 2; ++qt)
          if (act[qt]) S[qt][sb] = mfma(a, qf[qt][kk], kk == 0 ? float16v{} : S[qt][sb]);
      }
    }

    float mx[2];
    bool grow = false;
#pragma unroll
    for (int qt = 0; qt < 2; ++qt) {
      if (!act[qt]) continue;
      float16v& s0 = S[qt][0];
      float16v& s1 = S[qt][1];
      // Causal mask on tiles that reach past the query tile's first row.
      if (key0 + kBN - 1 > rq[qt]) {
        const int lim = rq[qt] + n - key0 - 8 * g;  // element i masked when 16*(i/8) + i%8 (+32) > lim
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const int k = 16 * (i >> 3) + (i & 7);
          if (k > lim) s0[i] = -INFINITY;
          if (k + 32 > lim) s1[i] = -INFINITY;
        }
      }
      // The tile's row maximum (raw scores; c > 0 keeps the order), both lane halves.
      float x = __builtin_fmaxf(s0[0], s1[0]);
#pragma unroll
      for (int i = 1; i < 16; ++i) x = __builtin_fmaxf(x, __builtin_fmaxf(s0[i], s1[i]));
      mx[qt] = __builtin_fmaxf(x, xlane(x, swapAddr)) * c;
      grow |= mx[qt] > m[qt] + kLazy;
    }

    // Move the reference only when some row of the wave outgrew it by kLazy.
    if (__builtin_amdgcn_ballot_w64(grow) != 0) {
#pragma unroll
      for (int qt = 0; qt < 2; ++qt) {
        if (!act[qt]) continue;
        const float m_new = __builtin_fmaxf(m[qt], mx[qt]);
        const float alpha = __builtin_amdgcn_exp2f(m[qt] - m_new);  // 0 on a row's first tile
        m[qt] = m_new;
        l[qt] *= alpha;
        o[qt][0] *= alpha;
        o[qt][1] *= alpha;
      }
    }

    // P = 2^(S c - m), rounded to binary16 for the product with V: slice ks
    // of query tile qt holds keys 16ks + 8g .. +7.
    half8 pb[2][4];
#pragma unroll
    for (int qt = 0; qt < 2; ++qt) {
      if (!act[qt]) continue;
      float16v& s0 = S[qt][0];
      float16v& s1 = S[qt][1];
      const float neg_m = -m[qt];
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        s0[i] = __builtin_amdgcn_exp2f(__builtin_fmaf(s0[i], c, neg_m));
        s1[i] = __builtin_amdgcn_exp2f(__builtin_fmaf(s1[i], c, neg_m));
      }
      pb[qt][0] = to_half8(__builtin_shufflevector(s0, s0, 0, 1, 2, 3, 4, 5, 6, 7));
      pb[qt][1] = to_half8(__builtin_shufflevector(s0, s0, 8, 9, 10, 11, 12, 13, 14, 15));
      pb[qt][2] = to_half8(__builtin_shufflevector(s1, s1, 0, 1, 2, 3, 4, 5, 6, 7));
      pb[qt][3] = to_half8(__builtin_shufflevector(s1, s1, 8, 9, 10, 11, 12, 13, 14, 15));
    }

    // O^T += V^T P^T over four 16-key slices, overlapping the row sums of P.
#pragma unroll
    for (int ks4 = 0; ks4 < 4; ++ks4) {
#pragma unroll
      for (int dt = 0; dt < 2; ++dt) {
        const half8 v = *reinterpret_cast<const half8*>(vs + vOff + 32 * dt * kRowHalfs + 16 * ks4);
#pragma unroll
        for (int qt = 0; qt < 2; ++qt)
          if (act[qt]) o[qt][dt] = mfma(v, pb[qt][ks4], o[qt][dt]);
      }
    }
#pragma unroll
    for (int qt = 0; qt < 2; ++qt) {
      if (!act[qt]) continue;
      float ls0 = S[qt][0][0], ls1 = S[qt][1][0];
#pragma unroll
      for (int i = 1; i < 16; ++i) {
        ls0 += S[qt][0][i];
        ls1 += S[qt][1][i];
      }
      l[qt] += ls0 + ls1;
    }
  };

  using T1 = std::integral_constant<bool, true>;
  using F0 = std::integral_constant<bool, false>;
  load_tile(0);
  store_tile(0);
  for (int j = 0; j < nkt; ++j) {
    const int buf = j & 1;
    if (j + 1 < nkt) load_tile(j + 1);
    __syncthreads();
    const bool a0 = j < need0, a1 = j < need1;
    if (a0 && a1)
      tile_body(T1{}, T1{}, j, buf);
    else if (a1)
      tile_body(F0{}, T1{}, j, buf);
    else if (a0)
      tile_body(T1{}, F0{}, j, buf);
    if (j + 1 < nkt) store_tile(buf ^ 1);
  }

  // Epilogue: the row sum over both lane halves, O / l, and m + log2 l.
#pragma unroll
  for (int qt = 0; qt < 2; ++qt) {
    if ((qt == 0 ? need0 : need1) == 0) continue;
    const int row = rq[qt] + n;
    const float lt = l[qt] + xlane(l[qt], swapAddr);
    const float inv = __builtin_amdgcn_rcpf(lt);
    const float lse = m[qt] + __builtin_amdgcn_logf(lt);
    if (row < T) {
      half_t* orow = O + (size_t)row * Hq * kD + (size_t)h * kD + 4 * g;
#pragma unroll
      for (int q4 = 0; q4 < 4; ++q4) {
        // accumulator elements 4q4 .. 4q4+3 are d = 8q4 + 4g + 0..3 (+32 in o[qt][1])
        const float16v& a = o[qt][0];
        const float16v& b = o[qt][1];
        const float4v va = {a[4 * q4], a[4 * q4 + 1], a[4 * q4 + 2], a[4 * q4 + 3]};
        const float4v vb = {b[4 * q4], b[4 * q4 + 1], b[4 * q4 + 2], b[4 * q4 + 3]};
        *reinterpret_cast<half4*>(orow + 8 * q4) = __builtin_convertvector(va * inv, half4);
        *reinterpret_cast<half4*>(orow + 32 + 8 * q4) = __builtin_convertvector(vb * inv, half4);
      }
      if (g == 0) L[(size_t)h * T + row] = lse;
    }
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
  constexpr int RS = kWaves / GW;
  const int G = Hq / Hkv;
  const int nBlocks = (T + 31) / 32;
  const int nPairs = (nBlocks + 1) / 2;
  const int nSlotGroups = (nPairs + RS - 1) / RS;
  const int nHeadGroups = G / GW;
  const unsigned grid = (unsigned)nSlotGroups * (unsigned)Hkv * (unsigned)nHeadGroups;
  hipLaunchKernelGGL((sattn_fwd_kernel<GW, VT_VEC>), dim3(grid), dim3(kThreads), 0, stream, Q, K,
                     Vt, O, L, c, T, Hq, Hkv, G, nBlocks, nPairs, nSlotGroups, nHeadGroups);
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
