// The materialised causal attention for gfx950 (CDNA4): the baseline the
// streaming forward avoids, with its C entry.
//
// What it computes (the pages' materialised path: the Graph page's scores
// plane, cgScores / cgScoresBytes, 4 H T^2 bytes, and its binary16 variant;
// the causal softmax device image of the Coppelius device-image page; the
// StreamingAttentionSM86 page's note that the materialised path rounds its
// probabilities to binary16 before their product with V):
//   1. scores:  S[h][i][j] = c (q_i . k_j), binary32, base-2 units, for j <= i;
//   2. softmax: L[h][i] = log2 sum_{j<=i} 2^S[h][i][j] and the probabilities
//      P[h][i][j] = 2^(S[h][i][j] - L[h][i]) rounded to binary16;
//   3. P V:     O[i][h*64 + d] = sum_{j<=i} P[h][i][j] V[j][d], binary32 sums,
//      rounded to binary16 (token-major, like the streaming forward's O).
// The planes hold T x T per head, so this path moves about 10 H T^2 bytes
// through HBM where the streaming forward moves the inputs and outputs only.
//
// gfx950 design:
//  * Scores: one workgroup per run of up to four 64 x 64 tiles of one tile
//    row (single tiles for small problems) on or below the diagonal (tiles above it are never touched), four
//    waves of 32 x 32, each one v_mfma_f32_32x32x16_f16 chain per tile over
//    the 64 head-width columns with its operands straight from global memory
//    (16-byte rows of Q, loaded once per run, and of K).  In the
//    accumulator a lane holds one key column, so the 32 lanes of a row store
//    128 consecutive bytes.  The stores bypass the caches' allocation
//    (non-temporal): the plane is written once and read back only by the
//    next launch, and write-allocating it in L2 halved the write rate.  Each
//    XCD takes a contiguous run of tiles (row by row), so a row's pieces
//    leave one L2.
//  * The softmax streams S in and P out the same way (non-temporal).
//  * Softmax: one wave per row, 4-float reads per lane; the row (up to 4096
//    keys) stays in registers while a running maximum and sum per lane are
//    merged across the wave, then P is written from the registers, so S is
//    read once; longer rows are read twice.  HBM-bound.
//  * P V: a workgroup takes 128 query rows of a head (a wave 32 rows x all
//    64 columns) and stages each 64-key V^T tile and the 128 x 64 tile of P
//    rows in LDS once for its four waves (coalesced loads; P swizzled so the
//    operand reads hit every bank once), with the next four tiles in flight
//    in four register sets (two when T % 8 != 0).  Keys past the row (only in the diagonal tile)
//    are masked in registers, so the planes' memory above the diagonal is
//    never read into a result.  O leaves through LDS as whole row segments.
#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>
#include <string.h>

#include <atomic>

#include "sattn.h"
#include "sattn_lds.h"

namespace {

typedef _Float16 half_t;
typedef _Float16 half4 __attribute__((ext_vector_type(4)));
typedef _Float16 half8 __attribute__((ext_vector_type(8)));
typedef float float4v __attribute__((ext_vector_type(4)));
typedef float float16v __attribute__((ext_vector_type(16)));

constexpr int kD = SATTN_HEAD_DIM;

__device__ __forceinline__ float16v mfma(half8 a, half8 b, float16v c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ half8 ld8(const half_t* p) { return *reinterpret_cast<const half8*>(p); }

// Workgroups are dealt to the eight XCDs round-robin by linear index.  This
// returns the workgroup's place (x fastest, then y) in an order where each
// XCD receives one contiguous run, so consecutive tiles of a plane's rows
// meet in one L2 before they go to HBM.
__device__ __forceinline__ int xcd_linear() {
  const int n = gridDim.x * gridDim.y, b = blockIdx.y * gridDim.x + blockIdx.x;
  const int xcd = b % 8, idx = b / 8;
  return xcd * (n / 8) + min(xcd, n % 8) + idx;
}

// -------------------------------------------------------------------------
// 1. scores.  Grid (chunks of the lower triangle, Hq), 256 threads.  A chunk
// is up to CH consecutive 64-key tiles of one 64-row tile row (CH = 4 when
// that still leaves many workgroups, else 1); wave w computes block
// (w / 2, w % 2) of each of them, with its 32 Q rows loaded once per chunk.
// -------------------------------------------------------------------------

// Chunks in tile rows 0 .. it-1 (row it has it / CH + 1 of them).
template <int CH>
__host__ __device__ inline long long chunks_before(int it) {
  const long long q = it / CH, r = it % CH;
  return it + (long long)CH * q * (q - 1) / 2 + q * r;
}

template <int CH>
__global__ void __launch_bounds__(256)
sattn_mat_scores_kernel(const half_t* __restrict__ Q, const half_t* __restrict__ K,
                        float* __restrict__ S, float c, int T, int G) {
  const int lin = xcd_linear();
  const int chunk = lin % gridDim.x, h = lin / gridDim.x, kv = h / G;
  // the tile row: the largest it with chunks_before(it) <= chunk
  int lo = 0, hi = (T + 63) / 64;
  while (hi - lo > 1) {
    const int mid = (lo + hi) >> 1;
    if (chunks_before<CH>(mid) <= chunk) lo = mid;
    else hi = mid;
  }
  const int it = lo;
  const int jt0 = (chunk - (int)chunks_before<CH>(it)) * CH, jt1 = min(jt0 + CH - 1, it);
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63, n = lane & 31, g = lane >> 5;
  const int i0 = it * 64 + 32 * (wave >> 1);
  const int ia = i0 + n;
  half8 qa[4];
#pragma unroll
  for (int kk = 0; kk < 4; ++kk)
    qa[kk] = ia < T ? ld8(Q + ((size_t)h * T + ia) * kD + 16 * kk + 8 * g) : half8{};
  __shared__ __attribute__((aligned(16))) float blk[4][32 * 36];
  float* const bw = blk[wave];
  const bool rowsAligned = (T & 3) == 0 && (reinterpret_cast<uintptr_t>(S) & 15) == 0;
  for (int jt = jt0; jt <= jt1; ++jt) {
    const int j0 = jt * 64 + 32 * (wave & 1);
    if (j0 > i0 + 31) continue;  // a 32 x 32 block wholly above the diagonal
    const int jb = j0 + n;
    float16v acc = {};
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) {
      const half8 b = jb < T ? ld8(K + ((size_t)kv * T + jb) * kD + 16 * kk + 8 * g) : half8{};
      acc = mfma(qa[kk], b, acc);
    }
    // element r of lane (n, g): query i0 + 8(r/4) + 4g + r%4, key jb
    if (j0 + 31 < i0 && j0 + 32 <= T && rowsAligned) {
      // wholly below the diagonal, all 32 keys inside T: the block goes
      // through the wave's LDS rows so that each store writes 16 bytes a
      // lane, eight whole 128-byte rows an instruction
#pragma unroll
      for (int r = 0; r < 16; ++r) bw[(8 * (r >> 2) + 4 * g + (r & 3)) * 36 + n] = acc[r] * c;
      // other lanes of this wave read what these wrote, and the next block
      // overwrites what they read: order the LDS accesses (a wave's LDS
      // operations complete in order, so this emits no wait)
      __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
      __builtin_amdgcn_wave_barrier();
      __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
      const int rr = lane >> 3, ch = lane & 7;
#pragma unroll
      for (int p = 0; p < 4; ++p) {  // rows 8p + lane/8, keys 4(lane%8) .. +3
        const int r = 8 * p + rr;
        const float4v v = *reinterpret_cast<const float4v*>(bw + r * 36 + 4 * ch);
        if (i0 + r < T)
          __builtin_nontemporal_store(
              v, reinterpret_cast<float4v*>(S + (size_t)h * T * T + (size_t)(i0 + r) * T + j0 + 4 * ch));
      }
      __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
      __builtin_amdgcn_wave_barrier();
      __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    } else if (jb < T) {
      float* col = S + (size_t)h * T * T + jb;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int i = i0 + 8 * (r >> 2) + 4 * g + (r & 3);
        if (i < T && jb <= i) __builtin_nontemporal_store(acc[r] * c, col + (size_t)i * T);
      }
    }
  }
}

// -------------------------------------------------------------------------
// 2. causal softmax.  One wave per row (h, i): 64 lanes x 4 keys per chunk.
// -------------------------------------------------------------------------
__device__ __forceinline__ void merge(float& m, float& l, float m2, float l2) {
  const float mn = fmaxf(m, m2);
  if (mn == -INFINITY) return;  // both empty
  l = l * __builtin_amdgcn_exp2f(m - mn) + l2 * __builtin_amdgcn_exp2f(m2 - mn);
  m = mn;
}

// Rows of at most 64 * 4 * NCH keys: the row stays in registers between the
// two passes, so S is read from HBM once.  NCH = 0: any length, two reads.
template <bool VEC, int NCH>
__global__ void __launch_bounds__(256)
sattn_mat_softmax_kernel(const float* __restrict__ S, half_t* __restrict__ P,
                         float* __restrict__ L, int T, int rows) {
  const int row = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (row >= rows) return;
  const int lane = threadIdx.x & 63;
  const int i = row % T;
  const int cnt = i + 1;  // keys 0..i
  const float* s = S + (size_t)row * T;
  half_t* p = P + (size_t)row * T;
  float m = -INFINITY, l = 0.0f;
  auto chunk = [&](int base, float (&v)[4]) {
    const int j = base + 4 * lane;
    if (VEC && j + 3 < cnt) {
      // read once when the row stays in registers (NCH > 0): stream it past L2
      const float4v x = NCH > 0 ? __builtin_nontemporal_load(reinterpret_cast<const float4v*>(s + j))
                                : *reinterpret_cast<const float4v*>(s + j);
#pragma unroll
      for (int e = 0; e < 4; ++e) v[e] = x[e];
    } else {
#pragma unroll
      for (int e = 0; e < 4; ++e) v[e] = j + e < cnt ? s[j + e] : -INFINITY;
    }
  };
  auto fold = [&](const float (&v)[4]) {
    const float mx = fmaxf(fmaxf(v[0], v[1]), fmaxf(v[2], v[3]));
    const float mn = fmaxf(m, mx);
    if (mn != -INFINITY) {
      float t = 0.0f;
#pragma unroll
      for (int e = 0; e < 4; ++e) t += __builtin_amdgcn_exp2f(v[e] - mn);
      l = l * __builtin_amdgcn_exp2f(m - mn) + t;
      m = mn;
    }
  };
  auto emit = [&](int base, const float (&v)[4], float lse) {
    const int j = base + 4 * lane;
    if (VEC && j + 3 < cnt) {
      half4 y;
#pragma unroll
      for (int e = 0; e < 4; ++e) y[e] = (half_t)__builtin_amdgcn_exp2f(v[e] - lse);
      __builtin_nontemporal_store(y, reinterpret_cast<half4*>(p + j));
    } else {
#pragma unroll
      for (int e = 0; e < 4; ++e)
        if (j + e < cnt) p[j + e] = (half_t)__builtin_amdgcn_exp2f(v[e] - lse);
    }
  };
  float keep[NCH > 0 ? NCH : 1][4];
  if constexpr (NCH > 0) {
#pragma unroll
    for (int cix = 0; cix < NCH; ++cix)
      if (cix * 256 < cnt) chunk(cix * 256, keep[cix]);
#pragma unroll
    for (int cix = 0; cix < NCH; ++cix)
      if (cix * 256 < cnt) fold(keep[cix]);
  } else {
    for (int base = 0; base < cnt; base += 256) {
      float v[4];
      chunk(base, v);
      fold(v);
    }
  }
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) {
    const float m2 = __shfl_xor(m, off, 64);
    const float l2 = __shfl_xor(l, off, 64);
    merge(m, l, m2, l2);
  }
  const float lse = m + __builtin_amdgcn_logf(l);
  if constexpr (NCH > 0) {
#pragma unroll
    for (int cix = 0; cix < NCH; ++cix)
      if (cix * 256 < cnt) emit(cix * 256, keep[cix], lse);
  } else {
    for (int base = 0; base < cnt; base += 256) {
      float v[4];
      chunk(base, v);
      emit(base, v, lse);
    }
  }
  if (lane == 0) L[row] = lse;
}

// -------------------------------------------------------------------------
// 3. P V.  Grid (ceil(T / 128) row blocks, heaviest first; Hq), 256 threads:
// wave w takes query rows 128 rb + 32 w .. +31 and all 64 head-width
// columns.  Per 64-key tile the workgroup stages the V^T tile and the
// 128 x 64 tile of P rows in LDS once (coalesced 16-byte loads, double-
// buffered); the waves take their P operands from the swizzled P tile.  Keys
// past a row (only in the diagonal tile) are masked in registers, so the
// plane's memory above the diagonal is never read into a result.
// -------------------------------------------------------------------------
constexpr int kRowHalfs = kD + 8;  // V^T tile row in LDS: 64 keys + 16 bytes of padding
constexpr int kBufferWord3 = 0x00020000;   // raw buffer, 32-bit data format
constexpr unsigned kOutOfRange = 0x7FFFFFF0u;  // a buffer offset past every range
constexpr int kTileHalfs = kD * kRowHalfs;
constexpr int kPTileHalfs = 128 * sattn_lds::kRowHalfs;  // P tile: 128 rows x 64 keys, swizzled

template <bool VEC>
__global__ void __launch_bounds__(256)
sattn_mat_pv_kernel(const half_t* __restrict__ P, const half_t* __restrict__ Vt,
                    half_t* __restrict__ O, int T, int Hq, int G, int nRowBlocks) {
  __shared__ __attribute__((aligned(16))) half_t vbuf[2 * kTileHalfs];
  __shared__ __attribute__((aligned(16))) half_t pbuf[2 * kPTileHalfs];
  const int h = blockIdx.y, kv = h / G;
  const int rb = nRowBlocks - 1 - (int)blockIdx.x;
  const int tid = threadIdx.x;
  const int wave = tid >> 6, lane = tid & 63, n = lane & 31, g = lane >> 5;
  const int row0 = rb * 128;
  const int i0 = row0 + 32 * wave;
  const int ia = i0 + n;
  const int nkt = (min(T, row0 + 128) - 1) / 64 + 1;  // key tiles of the workgroup
  const half_t* Vh = Vt + (size_t)kv * kD * T;
  const half_t* Ph = P + (size_t)h * T * T;
  // staging: thread t owns 16-byte chunks t and t + 256 of the V^T tile (row
  // d = c / 8, keys 8 (c % 8) ..) and chunks t + 256 k (k < 4) of the P tile
  // (row c / 8 of the block, keys 8 (c % 8) ..); rows past T, and keys past T
  // of a row, read as zeros
  const int cr = tid >> 3, cc = tid & 7;
  // With T % 8 == 0 the loads are buffer loads over the head's V^T and over
  // the workgroup's rows of P: a chunk lies wholly before or past T, rows past
  // T fall past the descriptor's range, and chunks past T take an offset past
  // it, so all read zeros without a branch (and the waits for one register
  // set leave the other in flight).
  const unsigned pRows = (unsigned)min(128, T - row0);
  const __amdgpu_buffer_rsrc_t vrsrc = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<half_t*>(Vh), 0, kD * T * 2, kBufferWord3);
  const __amdgpu_buffer_rsrc_t prsrc = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<half_t*>(Ph + (size_t)row0 * T), 0, (int)(pRows * (unsigned)T * 2u), kBufferWord3);
  auto load = [&](int kt, half8 (&st)[2], half8 (&sp)[4]) {
    const int key = kt * 64 + cc * 8;
    if constexpr (VEC) {
      // offsets stay below 2^28, so or-ing in kOutOfRange moves a chunk past T
      // out of range
      const unsigned oor = key < T ? 0u : kOutOfRange;
#pragma unroll
      for (int p = 0; p < 2; ++p) {
        const unsigned off = (((unsigned)(cr + 32 * p) * (unsigned)T + (unsigned)key) * 2u) | oor;
        st[p] = __builtin_bit_cast(half8, __builtin_amdgcn_raw_buffer_load_b128(vrsrc, off, 0, 0));
      }
#pragma unroll
      for (int p = 0; p < 4; ++p) {
        const unsigned off = (((unsigned)(cr + 32 * p) * (unsigned)T + (unsigned)key) * 2u) | oor;
        sp[p] = __builtin_bit_cast(half8, __builtin_amdgcn_raw_buffer_load_b128(prsrc, off, 0, 0));
      }
      return;
    }
#pragma unroll
    for (int p = 0; p < 2; ++p) {
      const int d = cr + 32 * p;
      {
#pragma unroll
        for (int e = 0; e < 8; ++e) st[p][e] = key + e < T ? Vh[(size_t)d * T + key + e] : (half_t)0;
      }
    }
#pragma unroll
    for (int p = 0; p < 4; ++p) {
      const int r = row0 + cr + 32 * p;
      const half_t* src = Ph + (size_t)min(r, T - 1) * T + key;
      {
#pragma unroll
        for (int e = 0; e < 8; ++e) sp[p][e] = (r < T && key + e < T) ? src[e] : (half_t)0;
      }
    }
  };
  auto store = [&](int buf, const half8 (&st)[2], const half8 (&sp)[4]) {
#pragma unroll
    for (int p = 0; p < 2; ++p)
      *reinterpret_cast<half8*>(vbuf + buf * kTileHalfs + (cr + 32 * p) * kRowHalfs + cc * 8) = st[p];
#pragma unroll
    for (int p = 0; p < 4; ++p)
      *reinterpret_cast<half8*>(pbuf + buf * kPTileHalfs + sattn_lds::chunk_offset(cr + 32 * p, cc)) = sp[p];
  };
  float16v acc0 = {}, acc1 = {};
  auto compute = [&](int kt, int buf) {
    if (kt * 64 <= i0 + 31 && i0 < T) {
      half8 a[4];
      const half_t* pb = pbuf + buf * kPTileHalfs;
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        a[u] = ld8(pb + sattn_lds::chunk_offset(32 * wave + n, 2 * u + g));
        if (kt * 64 + 63 > i0) {  // the diagonal tile: keys past the row are zero
          const int ja = kt * 64 + 16 * u + 8 * g;
#pragma unroll
          for (int e = 0; e < 8; ++e)
            if (ja + e > ia) a[u][e] = (half_t)0;
        }
      }
      const half_t* vb = vbuf + buf * kTileHalfs + n * kRowHalfs + 8 * g;
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        acc0 = mfma(a[u], ld8(vb + 16 * u), acc0);
        acc1 = mfma(a[u], ld8(vb + 32 * kRowHalfs + 16 * u), acc1);
      }
    }
  };
  // kSets tiles in flight: tile t is computed from LDS buffer t % 2 while
  // tiles t + 1 .. t + kSets wait or load in register set (t + i) % kSets.
  // The steps come in whole groups of kSets and every step issues the same
  // loads, stores and barrier (past the last tile they repeat it, unused), so
  // the wait for the oldest set leaves the newer ones in flight.
  constexpr int kSets = VEC ? 4 : 2;  // the element-wise loads of T % 8 != 0 need more registers
  half8 st[kSets][2], sp[kSets][4];
#pragma unroll
  for (int u = 0; u < kSets; ++u) load(min(u, nkt - 1), st[u], sp[u]);
  store(0, st[0], sp[0]);
  __syncthreads();
  for (int kt = 0; kt < nkt; kt += kSets) {
#pragma unroll
    for (int u = 0; u < kSets; ++u) {
      const int t = kt + u;
      // tile t + 1 goes into the buffer tile t - 1 left before the last
      // barrier, ahead of tile t's products so its stores complete under them
      store((u + 1) & 1, st[(u + 1) % kSets], sp[(u + 1) % kSets]);
      load(min(t + kSets, nkt - 1), st[u], sp[u]);
      if (t < nkt) compute(t, u & 1);
      __syncthreads();
    }
  }
  // Element r of lane (n, g) is query i0 + 8(r/4) + 4g + r%4, column n (acc0)
  // or 32 + n (acc1).  The wave's 32 rows go through its own LDS rows (the P
  // buffers are free once every wave has passed the last tile) so that each
  // store writes a whole 128-byte row segment with eight lanes.
  __syncthreads();
  if (i0 < T) {
    half_t* const ob = pbuf + wave * 32 * kRowHalfs;
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      half_t* const orow = ob + (8 * (r >> 2) + 4 * g + (r & 3)) * kRowHalfs;
      orow[n] = (half_t)acc0[r];
      orow[32 + n] = (half_t)acc1[r];
    }
    // other lanes of this wave read what these wrote (a wave's LDS operations
    // complete in order, so this emits no wait)
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    const int rr = lane >> 3, ch = lane & 7;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int r = 8 * q + rr;
      if (i0 + r < T)
        *reinterpret_cast<half8*>(O + (size_t)(i0 + r) * Hq * kD + (size_t)h * kD + 8 * ch) =
            ld8(ob + r * kRowHalfs + 8 * ch);
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

}  // namespace

namespace {

void launch_scores(const half_t* q, const half_t* k, float* S, float c, int T, int Hq, int Hkv,
                   hipStream_t strm) {
  // runs of four tiles per workgroup while that leaves at least 16 per CU
  const int nt = (T + 63) / 64;
  if (chunks_before<4>(nt) * Hq >= 16 * 256) {
    const unsigned chunks = (unsigned)chunks_before<4>(nt);
    hipLaunchKernelGGL(sattn_mat_scores_kernel<4>, dim3(chunks, (unsigned)Hq), dim3(256), 0,
                       strm, q, k, S, c, T, Hq / Hkv);
  } else {
    const unsigned chunks = (unsigned)chunks_before<1>(nt);
    hipLaunchKernelGGL(sattn_mat_scores_kernel<1>, dim3(chunks, (unsigned)Hq), dim3(256), 0,
                       strm, q, k, S, c, T, Hq / Hkv);
  }
}

template <bool VEC>
void launch_softmax_vec(const float* S, half_t* p, float* L, int T, int Hq, hipStream_t strm) {
  const int rows = Hq * T;
  const dim3 grid((unsigned)((rows + 3) / 4));
  if (T <= 1024)
    hipLaunchKernelGGL((sattn_mat_softmax_kernel<VEC, 4>), grid, dim3(256), 0, strm, S, p, L, T,
                       rows);
  else if (T <= 4096)
    hipLaunchKernelGGL((sattn_mat_softmax_kernel<VEC, 16>), grid, dim3(256), 0, strm, S, p, L, T,
                       rows);
  else
    hipLaunchKernelGGL((sattn_mat_softmax_kernel<VEC, 0>), grid, dim3(256), 0, strm, S, p, L, T,
                       rows);
}

void launch_softmax(const float* S, half_t* p, float* L, int T, int Hq, hipStream_t strm) {
  if (T % 4 == 0)
    launch_softmax_vec<true>(S, p, L, T, Hq, strm);
  else
    launch_softmax_vec<false>(S, p, L, T, Hq, strm);
}

void launch_pv(const half_t* p, const half_t* v, half_t* o, int T, int Hq, int Hkv,
               hipStream_t strm) {
  const int nrb = (T + 127) / 128;
  const dim3 grid((unsigned)nrb, (unsigned)Hq);
  if (T % 8 == 0)
    hipLaunchKernelGGL(sattn_mat_pv_kernel<true>, grid, dim3(256), 0, strm, p, v, o, T, Hq,
                       Hq / Hkv, nrb);
  else
    hipLaunchKernelGGL(sattn_mat_pv_kernel<false>, grid, dim3(256), 0, strm, p, v, o, T, Hq,
                       Hq / Hkv, nrb);
}

int launched() { return hipGetLastError() == hipSuccess ? SATTN_OK : SATTN_ERR_LAUNCH; }

}  // namespace

extern "C" int sattn_mat_fwd(const void* Q, const void* K, const void* Vt, void* O, float* L,
                             float* S, void* P, float c, int T, int Hq, int Hkv, void* stream) {
  const int st = sattn_mat_fwd_check(Q, K, Vt, O, L, S, P, c, T, Hq, Hkv);
  if (st != SATTN_OK) return st;
  const int dst = check_device();
  if (dst != SATTN_OK) return dst;
  const hipStream_t strm = static_cast<hipStream_t>(stream);
  half_t* p = static_cast<half_t*>(P);
  launch_scores(static_cast<const half_t*>(Q), static_cast<const half_t*>(K), S, c, T, Hq, Hkv,
                strm);
  launch_softmax(S, p, L, T, Hq, strm);
  launch_pv(p, static_cast<const half_t*>(Vt), static_cast<half_t*>(O), T, Hq, Hkv, strm);
  return launched();
}

extern "C" int sattn_mat_scores(const void* Q, const void* K, float* S, float c, int T, int Hq,
                                int Hkv, void* stream) {
  const int st = sattn_mat_scores_check(Q, K, S, c, T, Hq, Hkv);
  if (st != SATTN_OK) return st;
  const int dst = check_device();
  if (dst != SATTN_OK) return dst;
  launch_scores(static_cast<const half_t*>(Q), static_cast<const half_t*>(K), S, c, T, Hq, Hkv,
                static_cast<hipStream_t>(stream));
  return launched();
}

extern "C" int sattn_mat_softmax(const float* S, void* P, float* L, int T, int Hq,
                                 void* stream) {
  const int st = sattn_mat_softmax_check(S, P, L, T, Hq);
  if (st != SATTN_OK) return st;
  const int dst = check_device();
  if (dst != SATTN_OK) return dst;
  launch_softmax(S, static_cast<half_t*>(P), L, T, Hq, static_cast<hipStream_t>(stream));
  return launched();
}

extern "C" int sattn_mat_pv(const void* P, const void* Vt, void* O, int T, int Hq, int Hkv,
                            void* stream) {
  const int st = sattn_mat_pv_check(P, Vt, O, T, Hq, Hkv);
  if (st != SATTN_OK) return st;
  const int dst = check_device();
  if (dst != SATTN_OK) return dst;
  launch_pv(static_cast<const half_t*>(P), static_cast<const half_t*>(Vt), static_cast<half_t*>(O),
            T, Hq, Hkv, static_cast<hipStream_t>(stream));
  return launched();
}
