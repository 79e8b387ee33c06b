// Stable grouping of the N = T*k (token, slot) pairs by expert, and the row
// gather. Integer-only and atomic-free, so the result is exact and identical
// on every run.
//
// The faster-moe page (Unsloth, "Fine-tune MoE models 12x faster", section
// "What is torch._grouped_mm?") walks, per expert, the tokens routed to it;
// a grouped GEMM needs those rows contiguous, expert after expert. This is a
// counting sort keyed by expert, stable in pair order p = t*k + j:
//
//   1. hist     one wave per 64-pair chunk: ballot-built peer masks give each
//               pair its rank among same-expert pairs of the chunk and each
//               expert its chunk count -> table[e][chunk]
//   2. colscan  one block per expert: exclusive scan of its chunk counts
//               (in place) and the expert's total -> counts[e]
//   3. offsets  one block: exclusive scan of counts -> offsets[E+1]
//   4. scatter  one wave per chunk: pos = offsets[e] + table[e][chunk] + rank
//   5. gather   X_perm[pos] = x[sorted_pair[pos] / k], 16-byte vectors
//
// Pairs whose expert id lies outside [0, E) (a caller error) are dropped:
// they get inv_pos = -1 and no row, and every access stays in bounds.
#include <mutex>

#include "device_common.h"
#include "launch.h"

namespace moe {

namespace {

constexpr int kChunk = 64;          // pairs per chunk = one wave
constexpr int kWavesPerBlock = 4;

// Peer mask: lanes whose key equals this lane's key (keys < 2^11).
__device__ __forceinline__ uint64_t peer_mask(int key) {
  uint64_t m = ~0ull;
#pragma unroll
  for (int b = 0; b < 11; ++b) {
    uint64_t bal = __ballot((key >> b) & 1);
    m &= ((key >> b) & 1) ? bal : ~bal;
  }
  return m;
}

__device__ __forceinline__ int expert_of(const int32_t* ids, int64_t p, int64_t N, int E) {
  if (p >= N) return 1024 + 1;  // padding lane: key no real expert has
  int e = ids[p];
  return (e >= 0 && e < E) ? e : 1024 + 2;
}

// table: [E][nchunks] int32
__global__ __launch_bounds__(256) void hist_kernel(const int32_t* __restrict__ ids, int64_t N,
                                                   int E, int nchunks,
                                                   int32_t* __restrict__ table) {
  __shared__ int32_t cnt[kWavesPerBlock][1024];
  const int wave = threadIdx.x / kWave, lane = threadIdx.x & (kWave - 1);
  const int chunk0 = blockIdx.x * kWavesPerBlock;
  for (int i = threadIdx.x; i < kWavesPerBlock * E; i += blockDim.x)
    cnt[i / E][i % E] = 0;
  __syncthreads();
  const int chunk = chunk0 + wave;
  if (chunk < nchunks) {
    const int64_t p = static_cast<int64_t>(chunk) * kChunk + lane;
    const int e = expert_of(ids, p, N, E);
    const uint64_t m = peer_mask(e);
    const uint64_t below = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
    if (e < E && (m & below) == 0) cnt[wave][e] = __popcll(m);
  }
  __syncthreads();
  for (int i = threadIdx.x; i < kWavesPerBlock * E; i += blockDim.x) {
    const int w = i / E, e = i % E;
    if (chunk0 + w < nchunks) table[static_cast<int64_t>(e) * nchunks + chunk0 + w] = cnt[w][e];
  }
}

// Block-wide exclusive scan of one int per thread (256 threads). Returns the
// thread's exclusive prefix; *total gets the block sum.
__device__ __forceinline__ int block_exclusive_scan(int v, int* total) {
  __shared__ int wsum[256 / kWave];
  const int lane = threadIdx.x & (kWave - 1), wave = threadIdx.x / kWave;
  int incl = v;
#pragma unroll
  for (int off = 1; off < kWave; off <<= 1) {
    int o = __shfl_up(incl, off, kWave);
    if (lane >= off) incl += o;
  }
  if (lane == kWave - 1) wsum[wave] = incl;
  __syncthreads();
  int base = 0, tot = 0;
#pragma unroll
  for (int w = 0; w < 256 / kWave; ++w) {
    int s = wsum[w];
    if (w < wave) base += s;
    tot += s;
  }
  __syncthreads();
  *total = tot;
  return base + incl - v;
}

__global__ __launch_bounds__(256) void colscan_kernel(int32_t* __restrict__ table, int nchunks,
                                                      int32_t* __restrict__ counts) {
  const int e = blockIdx.x;
  int32_t* col = table + static_cast<int64_t>(e) * nchunks;
  constexpr int kItems = 4;
  int carry = 0;
  for (int base = 0; base < nchunks; base += 256 * kItems) {
    int v[kItems];
    int sum = 0;
#pragma unroll
    for (int i = 0; i < kItems; ++i) {
      int idx = base + threadIdx.x * kItems + i;
      v[i] = idx < nchunks ? col[idx] : 0;
      sum += v[i];
    }
    int tot;
    int pre = block_exclusive_scan(sum, &tot) + carry;
#pragma unroll
    for (int i = 0; i < kItems; ++i) {
      int idx = base + threadIdx.x * kItems + i;
      if (idx < nchunks) col[idx] = pre;
      pre += v[i];
    }
    carry += tot;
  }
  if (threadIdx.x == 0) counts[e] = carry;
}

// One block of 1024 threads: offsets[0..E] from counts[0..E-1] (E <= 1024).
__global__ __launch_bounds__(1024) void offsets_kernel(const int32_t* __restrict__ counts, int E,
                                                       int32_t* __restrict__ offsets) {
  __shared__ int wsum[1024 / kWave];
  const int lane = threadIdx.x & (kWave - 1), wave = threadIdx.x / kWave;
  int v = threadIdx.x < E ? counts[threadIdx.x] : 0;
  int incl = v;
#pragma unroll
  for (int off = 1; off < kWave; off <<= 1) {
    int o = __shfl_up(incl, off, kWave);
    if (lane >= off) incl += o;
  }
  if (lane == kWave - 1) wsum[wave] = incl;
  __syncthreads();
  int base = 0;
  for (int w = 0; w < wave; ++w) base += wsum[w];
  if (threadIdx.x < E) offsets[threadIdx.x] = base + incl - v;
  if (threadIdx.x == E - 1) offsets[E] = base + incl;
}

__global__ __launch_bounds__(256) void scatter_kernel(const int32_t* __restrict__ ids, int64_t N,
                                                      int E, int nchunks,
                                                      const int32_t* __restrict__ table,
                                                      const int32_t* __restrict__ offsets,
                                                      int32_t* __restrict__ sorted_pair,
                                                      int32_t* __restrict__ inv_pos) {
  const int lane = threadIdx.x & (kWave - 1);
  const int chunk = (blockIdx.x * blockDim.x + threadIdx.x) / kWave;
  if (chunk >= nchunks) return;
  const int64_t p = static_cast<int64_t>(chunk) * kChunk + lane;
  const int e = expert_of(ids, p, N, E);
  const uint64_t m = peer_mask(e);
  const uint64_t below = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
  if (p < N) {
    if (e < E) {
      const int rank = __popcll(m & below);
      const int pos = offsets[e] + table[static_cast<int64_t>(e) * nchunks + chunk] + rank;
      sorted_pair[pos] = static_cast<int32_t>(p);
      inv_pos[p] = pos;
    } else {
      inv_pos[p] = -1;
    }
  }
}

// X_perm[pos] = x[sorted_pair[pos] / k]; one thread per 16-byte chunk. The
// chunk index is split into (row, chunk) with 32-bit unsigned arithmetic (a
// 64-bit division costs about ten times as many instructions, a large share
// of this kernel's issue; the layer's shape limit keeps X_perm under 32 GiB,
// so its chunk count fits).
// NT: non-temporal stores, for an X_perm larger than the 256 MB Infinity
// Cache. One that fits is left in the cache for its next readers (the side
// product and the gate_up GEMM); a larger one would only evict their operands
// (Qwen3-shaped layer, 537 MB: side product -16%, layer step -1.6%; at
// gpt-oss shape, 189 MB, the same stores slow the side product by 17%).
template <bool NT>
__global__ __launch_bounds__(256) void gather_kernel(const uint4* __restrict__ x,
                                                     const int32_t* __restrict__ sorted_pair,
                                                     const int32_t* __restrict__ offsets, int E,
                                                     int k, uint32_t chunks_per_row,
                                                     uint4* __restrict__ xp) {
  typedef uint32_t Idx;
  const Idx g = static_cast<Idx>(blockIdx.x) * blockDim.x + threadIdx.x;
  const Idx rows = static_cast<Idx>(offsets[E]);
  const Idx pos = g / chunks_per_row, c = g - pos * chunks_per_row;
  if (pos >= rows) return;
  const Idx t = static_cast<Idx>(sorted_pair[pos]) / static_cast<Idx>(k);
  typedef unsigned int v4u __attribute__((ext_vector_type(4)));
  const v4u v = reinterpret_cast<const v4u*>(x)[static_cast<int64_t>(t) * chunks_per_row + c];
  v4u* dst = reinterpret_cast<v4u*>(xp) + static_cast<int64_t>(pos) * chunks_per_row + c;
  if constexpr (NT) __builtin_nontemporal_store(v, dst);
  else *dst = v;
}

}  // namespace

// The histogram table of moe_permute_noalloc: a file-scope device array (one
// copy per GPU the library runs on). In host code `scratch` names a
// host-side stand-in, not device memory: kernels get the address that
// hipGetSymbolAddress returns for the current GPU, looked up once per GPU.
static __device__ __align__(256) char scratch[MOE_PERMUTE_NOALLOC_BYTES];

namespace {
constexpr int kMaxDevices = 64;
std::mutex g_noalloc_mu;
void* g_noalloc_ptr[kMaxDevices] = {};
}  // namespace

hipError_t noalloc_permute_table(int32_t** table) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lk(g_noalloc_mu);
  if (!g_noalloc_ptr[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    g_noalloc_ptr[dev] = p;
  }
  *table = static_cast<int32_t*>(g_noalloc_ptr[dev]);
  return hipSuccess;
}

size_t permute_ws_bytes(int64_t N, int E) {
  const int64_t nchunks = (N + kChunk - 1) / kChunk;
  return static_cast<size_t>(nchunks) * E * sizeof(int32_t);
}

hipError_t launch_permute(const int32_t* ids, int64_t N, int E, int32_t* counts,
                          int32_t* offsets, int32_t* sorted_pair, int32_t* inv_pos,
                          int32_t* table, hipStream_t s, KernelTimer* tm) {
  const int nchunks = static_cast<int>((N + kChunk - 1) / kChunk);
  TimedScope scope(tm, MOE_K_PERMUTE, s);
  hipLaunchKernelGGL(hist_kernel, dim3((nchunks + kWavesPerBlock - 1) / kWavesPerBlock),
                     dim3(256), 0, s, ids, N, E, nchunks, table);
  hipLaunchKernelGGL(colscan_kernel, dim3(E), dim3(256), 0, s, table, nchunks, counts);
  hipLaunchKernelGGL(offsets_kernel, dim3(1), dim3(1024), 0, s, counts, E, offsets);
  hipLaunchKernelGGL(scatter_kernel, dim3((nchunks + kWavesPerBlock - 1) / kWavesPerBlock),
                     dim3(256), 0, s, ids, N, E, nchunks, table, offsets, sorted_pair, inv_pos);
  return hipGetLastError();
}

hipError_t launch_gather(const void* x, const int32_t* sorted_pair, const int32_t* offsets,
                         int E, int k, int64_t N, int64_t row_bytes, void* x_perm,
                         hipStream_t s, KernelTimer* tm) {
  const int64_t cpr = row_bytes / 16;
  const int64_t total = N * cpr;
  const dim3 grid(static_cast<unsigned>((total + 255) / 256));
  TimedScope scope(tm, MOE_K_GATHER, s);
  const bool nt = N * row_bytes > (int64_t{256} << 20);
  if (total + 255 > 0xffffffffLL) return hipErrorInvalidValue;  // excluded by the shape limit
  const uint4* xs = static_cast<const uint4*>(x);
  uint4* xd = static_cast<uint4*>(x_perm);
  if (!nt)
    hipLaunchKernelGGL((gather_kernel<false>), grid, dim3(256), 0, s, xs, sorted_pair, offsets, E,
                       k, static_cast<uint32_t>(cpr), xd);
  else
    hipLaunchKernelGGL((gather_kernel<true>), grid, dim3(256), 0, s, xs, sorted_pair, offsets, E,
                       k, static_cast<uint32_t>(cpr), xd);
  return hipGetLastError();
}

}  // namespace moe
