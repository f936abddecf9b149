// 2:4 SpMM for skinny column-major dense operands (C <= 32, the decode regime) with the
// reduction split across workgroups ("2:4 sparsity on sparse tensor cores", lecture notes:
// small products are bound by memory traffic and fixed costs).
//
// Why a split: with one workgroup per 16-row tile and all of K, every workgroup reads the
// whole dense operand (256 KiB at K = 4096, C = 32) from L2 to use it once, 3.5x the bytes
// of its share of the compressed weights. Here each wave applies every B operand it loads
// to RT = 4 row tiles (2 when fewer than 256 row tiles exist), which divides the B bytes
// per row by RT; the K range is cut into S <= 4 splits so that the grid still holds about
// one workgroup per CU.
//
//   * workgroup (g, s): rows [16 RT g, +16 RT), 64-position chunks [s Q, min(KC, (s+1) Q))
//     with Q = ceil(KC / S); its NW waves take the chunks round-robin.
//   * A is the operand-major storage: block (row tile, chunk) is one contiguous 1 KiB of
//     values and 128 B of metadata, loaded straight into the sparse-MFMA operands.
//   * B column-major: each lane loads its operand half (eight consecutive k of one
//     column); the four lanes of a column read whole 128-byte lines.
//   * the NW wave partials are summed through LDS; the workgroup (S >= 2) stores its fp32
//     tile in the workspace, publishes it with one agent-scope release fence and counts
//     itself in on the row group's counter; the workgroup that arrives last reads the S
//     tiles back, adds them in split order (so the result does not depend on the arrival
//     order), writes Y and sets the counter back to zero.
//   * the last workgroup also zeroes the S partial tiles it consumed, so a call leaves the
//     whole workspace zero. Where the counters end and the partial tiles begin depends on
//     the shape; without this, a later call of another shape on the same workspace would
//     take stale partial sums for its counters.
#include "device_common.hpp"
#include "launch.hpp"
#include "variant.hpp"
#include "validate.hpp"

#include <atomic>
#include <mutex>

namespace snm {

namespace {

constexpr int kSplitWaves = 16;           // as assumed by splitk_plan

struct SplitArgs {
  const uint16_t* values;   // operand-major values
  const uint8_t* meta;      // operand-major metadata
  const uint16_t* B;        // column-major: element (k, c) at B[c*ldb + k]
  uint16_t* Y;
  float* part;              // S x (G * 16 RT) x CP fp32 partial tiles
  uint32_t* count;          // G arrival counters, zero between calls
  int64_t R, K, C, ldb, ldy;
  int64_t KC, RT16;         // 64-position chunks; 16-row tiles of the padded storage
  int64_t G;                // row groups of 16 RT rows
  int S, Q;                 // splits; chunks per split
  int b_vec;                // B columns 16-byte aligned (ldb % 8 == 0, B 16-byte aligned)
};

// U chunks per wave and round: every load of a round is in flight before its first MFMA
// (U = 1 with four row tiles keeps the operands within the 128 VGPRs of 16-wave groups;
// 8-wave groups with U = 2 or 4 measured slower on MI355X).
template <int CP, int RT, int U, int NWAVES, bool BVEC>
__global__ void __launch_bounds__(64 * NWAVES)
k_spmm_nm_splitk(SplitArgs a) {
  constexpr int CT = CP / 16;
  extern __shared__ __align__(16) uint8_t smem[];
  __shared__ uint32_t last_flag;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int w = tid >> 6;
  constexpr int NW = NWAVES;
  const int q = lane >> 4;
  const int li = lane & 15;
  const int64_t g = blockIdx.x;
  const int s = blockIdx.y;
  const int64_t c_begin = (int64_t)s * a.Q;
  const int64_t c_end = c_begin + a.Q < a.KC ? c_begin + a.Q : a.KC;

  f4 acc[RT][CT];
#pragma unroll
  for (int i = 0; i < RT; ++i)
#pragma unroll
    for (int ct = 0; ct < CT; ++ct) acc[i][ct] = f4{0.f, 0.f, 0.f, 0.f};

  for (int64_t c0 = c_begin + w; c0 < c_end; c0 += U * NW) {
    h8 av[U][RT];
    uint32_t ai[U][RT];
    h16 bf[U][CT];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int64_t kc = c0 + u * NW;
      const bool live = kc < c_end;
#pragma unroll
      for (int i = 0; i < RT; ++i) {
        const int64_t rt = g * RT + i;
        h8 v = {};
        uint32_t id = 0;
        if (live && rt < a.RT16) {
          const int64_t blk = rt * a.KC + kc;
          v = *reinterpret_cast<const h8*>(a.values + blk * 512 + lane * 8);
          id = *reinterpret_cast<const uint16_t*>(a.meta + (blk * 64 + lane) * 2);
        }
        av[u][i] = v;
        ai[u][i] = id;
      }
      // B operand: column 16 ct + li, rows k1 + [0, 8) and k1 + 32 + [0, 8). K is a
      // multiple of 16 and k1 of 8, so each 8-row half lies wholly inside or outside K.
      const int64_t k1 = kc * 64 + 8 * q;
#pragma unroll
      for (int ct = 0; ct < CT; ++ct) {
        const int64_t col = 16 * ct + li;
        const uint16_t* colp = a.B + col * a.ldb;
        h8 lo = {}, hi = {};
        if (live && col < a.C) {
          if constexpr (BVEC) {
            if (k1 < a.K) lo = *reinterpret_cast<const h8*>(colp + k1);
            if (k1 + 32 < a.K) hi = *reinterpret_cast<const h8*>(colp + k1 + 32);
          } else {
#pragma unroll
            for (int e = 0; e < 8; ++e) {
              if (k1 < a.K) lo[e] = bits_f16(colp[k1 + e]);
              if (k1 + 32 < a.K) hi[e] = bits_f16(colp[k1 + 32 + e]);
            }
          }
        }
#pragma unroll
        for (int e = 0; e < 8; ++e) { bf[u][ct][e] = lo[e]; bf[u][ct][8 + e] = hi[e]; }
      }
    }
#pragma unroll
    for (int u = 0; u < U; ++u)
#pragma unroll
      for (int i = 0; i < RT; ++i)
#pragma unroll
        for (int ct = 0; ct < CT; ++ct) acc[i][ct] = smfmac16<0>(av[u][i], bf[u][ct], acc[i][ct], ai[u][i]);
  }

  // ---- sum the NW wave tiles through LDS: red[w][i][ct][lane] -------------------------
  f4* red = reinterpret_cast<f4*>(smem);
#pragma unroll
  for (int i = 0; i < RT; ++i)
#pragma unroll
    for (int ct = 0; ct < CT; ++ct) red[((w * RT + i) * CT + ct) * 64 + lane] = acc[i][ct];
  __syncthreads();
  constexpr int kTile = 16 * RT * CP;                 // fp32 elements of the workgroup tile
  constexpr int kPer = (kTile + 64 * NWAVES - 1) / (64 * NWAVES);
  const float* rp = reinterpret_cast<const float*>(red);
  float v[kPer];
#pragma unroll
  for (int j = 0; j < kPer; ++j) {
    const int e = tid + j * 64 * NW;
    float sum = 0.f;
    if (e < kTile) {
      const int r = e / CP;                            // row within the group
      const int c = e - r * CP;
      const int i = r >> 4, rr = r & 15, ct = c >> 4;
      const int ln = ((rr >> 2) << 4) | (c & 15);
      for (int ww = 0; ww < NW; ++ww) sum += rp[(((ww * RT + i) * CT + ct) * 64 + ln) * 4 + (rr & 3)];
    }
    v[j] = sum;
  }
  const int64_t row0 = g * 16 * RT;

  float* mine = a.part + ((int64_t)s * a.G + g) * kTile;
#pragma unroll
  for (int j = 0; j < kPer; ++j) {
    const int e = tid + j * 64 * NW;
    if (e < kTile) mine[e] = v[j];
  }
  // Every wave's stores have reached L2 before the barrier; one thread then publishes the
  // tile at agent scope and counts in. An agent-scope release writes back the XCD's L2 and
  // an acquire invalidates it, so each is issued once per workgroup, not once per thread
  // (once per thread measured 94 us per launch).
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  __syncthreads();
  if (tid == 0) {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "agent");
    const bool last = atomicAdd(a.count + g, 1u) == (uint32_t)(a.S - 1);
    if (last) __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");   // the other splits' tiles
    last_flag = last ? 1u : 0u;
  }
  __syncthreads();
  if (last_flag == 0u) return;
#pragma unroll
  for (int j = 0; j < kPer; ++j) {
    const int e = tid + j * 64 * NW;
    if (e >= kTile) continue;
    float t = 0.f;
    for (int ss = 0; ss < a.S; ++ss) {
      float* p = a.part + ((int64_t)ss * a.G + g) * kTile + e;
      t += ss == s ? v[j] : *p;
      *p = 0.f;   // every byte a call writes is zero again when it ends (see below)
    }
    v[j] = t;
  }
  if (tid == 0) __hip_atomic_store(a.count + g, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
#pragma unroll
  for (int j = 0; j < kPer; ++j) {
    const int e = tid + j * 64 * NW;
    if (e >= kTile) continue;
    const int r = e / CP;
    const int c = e - r * CP;
    const int64_t orow = row0 + r;
    if (orow < a.R && c < a.C) a.Y[orow * a.ldy + c] = f16_bits(to_f16(v[j]));
  }
}

// ---- the no-allocation variant's scratch ----------------------------------------------
// One array per device for the split reduction's counters and partial tiles, used by
// snm_spmm_nm_tiled_noalloc instead of a caller's workspace. In host code `scratch` names
// a host-side stand-in, not device memory: its device address comes from
// hipGetSymbolAddress, once per device, and only that address is ever handed to a kernel.
static __device__ __align__(256) uint8_t scratch[kSplitScratchBytes];

__global__ void __launch_bounds__(256) k_zero_scratch(u4* p, int64_t n16) {
  for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < n16; i += (int64_t)gridDim.x * 256)
    p[i] = u4{0u, 0u, 0u, 0u};
}

std::mutex g_scratch_mu;
void* g_scratch_ptr[64];
std::atomic<uint64_t> g_scratch_ready{0};   // bit d: device d's address is known and its
                                            // zero fill has been enqueued

// Device address of the current device's scratch. The first call on a device looks the
// array up and enqueues a fill kernel on `stream` (a kernel, not a memset, so that it can
// also be recorded into a graph) ahead of the caller's work; split calls then leave every
// byte they write zero, so the array stays zero between calls.
hipError_t scratch_of_current_device(void** out, hipStream_t stream) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= 64) return hipErrorInvalidDevice;
  const uint64_t bit = (uint64_t)1 << dev;
  if (!(g_scratch_ready.load(std::memory_order_acquire) & bit)) {
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (!(g_scratch_ready.load(std::memory_order_relaxed) & bit)) {
      void* p = nullptr;
      e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
      if (e != hipSuccess) return e;
      if (p == nullptr || ((uintptr_t)p & 255u) != 0) return hipErrorInvalidSymbol;
      hipLaunchKernelGGL(k_zero_scratch, dim3(256), dim3(256), 0, stream, (u4*)p,
                         (int64_t)(kSplitScratchBytes / 16));
      if ((e = hipGetLastError()) != hipSuccess) return e;
      g_scratch_ptr[dev] = p;
      g_scratch_ready.fetch_or(bit, std::memory_order_release);
    }
  }
  *out = g_scratch_ptr[dev];
  return hipSuccess;
}

}  // namespace

template <int CP, int RT, int U, bool BVEC>
static hipError_t launch_splitk(const SplitArgs& a, hipStream_t stream) {
  constexpr int nw = kSplitWaves;
  const size_t lds = (size_t)nw * RT * (CP / 16) * 64 * 16;
  auto kern = k_spmm_nm_splitk<CP, RT, U, nw, BVEC>;
  static std::atomic<uint64_t> lds_set{0};
  if (hipError_t e = ensure_lds_limit(lds_set, (const void*)kern, (int)lds)) return e;
  hipLaunchKernelGGL(kern, dim3((unsigned)a.G, (unsigned)a.S), dim3(64 * nw), lds, stream, a);
  return hipGetLastError();
}

hipError_t launch_spmm_nm_tiled_splitk(const void* values_t, const void* meta_t, int64_t R, int64_t K,
                                       const void* B, int64_t C, int64_t ldb, void* Y, int64_t ldy,
                                       void* workspace, hipStream_t stream) {
  const SplitPlan p = splitk_plan(R, K, C);
  if (p.splits < 2 || forced_variant() == Variant::kUnsplit) {
    // the split does not pay here: one workgroup per row tile, all of K
    log_variant("spmm_nm_tiled_ws", R, K, C, skinny_ring_selected(K, B, C, ldb, 1, true) ? "skinny ring" : "skinny");
    return launch_spmm_nm_tiled_skinny(values_t, meta_t, R, K, B, C, ldb, 1, Y, ldy, stream);
  }
  log_variant("spmm_nm_tiled_ws", R, K, C, p.splits == 2 ? "split 2" : p.splits == 3 ? "split 3" : "split 4");
  SplitArgs a{};
  a.values = (const uint16_t*)values_t;
  a.meta = (const uint8_t*)meta_t;
  a.B = (const uint16_t*)B;
  a.Y = (uint16_t*)Y;
  a.count = (uint32_t*)workspace;
  a.part = (float*)((uint8_t*)workspace + p.count_bytes);
  a.R = R; a.K = K; a.C = C; a.ldb = ldb; a.ldy = ldy;
  a.KC = (K + 63) / 64;
  a.RT16 = (R + 15) / 16;
  a.G = p.groups;
  a.S = p.splits;
  a.Q = p.chunks_per_split;
  a.b_vec = (ldb % 8 == 0) && (((uintptr_t)B & 15) == 0);
  if (p.rt == 4) {
    if (p.cp == 16)
      return a.b_vec ? launch_splitk<16, 4, 1, true>(a, stream) : launch_splitk<16, 4, 1, false>(a, stream);
    return a.b_vec ? launch_splitk<32, 4, 1, true>(a, stream) : launch_splitk<32, 4, 1, false>(a, stream);
  }
  if (p.cp == 16)
    return a.b_vec ? launch_splitk<16, 2, 2, true>(a, stream) : launch_splitk<16, 2, 2, false>(a, stream);
  return a.b_vec ? launch_splitk<32, 2, 2, true>(a, stream) : launch_splitk<32, 2, 2, false>(a, stream);
}

hipError_t launch_spmm_nm_tiled_splitk_noalloc(const void* values_t, const void* meta_t, int64_t R,
                                               int64_t K, const void* B, int64_t C, int64_t ldb,
                                               void* Y, int64_t ldy, hipStream_t stream) {
  const SplitPlan p = splitk_plan(R, K, C);
  void* ws = nullptr;
  if (p.splits >= 2 && forced_variant() != Variant::kUnsplit) {   // the unsplit kernel needs no scratch
    if (p.workspace_bytes > kSplitScratchBytes) return hipErrorInvalidValue;
    hipError_t e = scratch_of_current_device(&ws, stream);
    if (e != hipSuccess) return e;
  }
  return launch_spmm_nm_tiled_splitk(values_t, meta_t, R, K, B, C, ldb, Y, ldy, ws, stream);
}

}  // namespace snm
