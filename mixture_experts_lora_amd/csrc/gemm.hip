// Grouped expert GEMMs of the MoE-LoRA layer: forward and backward.
//
// Per expert e, over its rows X (permuted, expert after expert):
//   forward   h     = X W_gu^T + (s X A_gu^T) B_gu^T       act = silu(h_gate) h_up
//             y_exp = act W_d^T + (s act A_d^T) B_d^T
//   backward  dAct  = G W_d + (s G B_d) A_d                dH = SwiGLU'(h) dAct
//             dX    = dH W_gu + (s dH B_gu) A_gu
//             dB_d  = G^T (s act A_d^T)   dA_d  = (s G B_d)^T act
//             dB_gu = dH^T (s X A_gu^T)   dA_gu = (s dH B_gu)^T X
// The adapter is always applied in the split order (input times A, then B)
// and W + s B A is never formed (Unsloth, "Fine-tune MoE models 12x faster",
// faster-moe page, section "Faster LoRA MoE training"; the LoRA shapes and
// the frozen base weights are in its section "Implementation details"; the
// per-expert loop and the gate/up halves of gate_up_proj in its section
// "What is torch._grouped_mm?"). SwiGLU follows the fused LoRA MLP
// definition in the aiflowlearn.net Unsloth tutorial.
//
// One kernel template covers every product:
//  - GROUP_M: output rows are an expert's rows. A device-built tile list maps
//    each M tile to (expert, first row, valid rows); group sizes never leave
//    the device. The rank-r LoRA term is a second K segment appended to the
//    main K loop ([X | s X A^T] times [W | B]^T), so it costs one extra
//    K step and no extra pass over the output.
//  - GROUP_K: the reduction runs over an expert's rows (the LoRA weight
//    gradients), one block per (expert, M tile, N tile), so no atomics and
//    bit-identical results run to run.
// Operands are staged through LDS with k contiguous. Operands stored with k
// contiguous (activations; forward weights) are copied as 16-byte chunks;
// operands stored with the output dimension contiguous (backward weights,
// and both operands of the weight gradients) are transposed in registers in
// 4x8 blocks on their way into LDS. bf16 products use the gfx950
// v_mfma_f32_32x32x16_bf16 instruction with float32 accumulation; the
// weight tile is the MFMA A operand so that each lane ends up holding four
// consecutive output columns of one row (8-byte stores). float32 layers use a
// plain FMA kernel with the same tiling logic.
#include "device_common.h"
#include "launch.h"

namespace moe {

namespace {

enum Mode { GROUP_M = 0, GROUP_K = 1 };
enum Epi { EPI_STORE = 0, EPI_SWIGLU = 1, EPI_SWIGLU_BWD = 2 };

struct Opnd {
  const void* ptr;
  int64_t estride;  // elements between consecutive experts (0: not per expert)
  int64_t ld;       // leading dimension in elements
  int kcontig;      // 1: (mn, k) at ptr[mn*ld + k]; 0: at ptr[k*ld + mn]
  int vec;          // 16-byte chunks allowed (alignment and extents are multiples of 8)
};

struct GemmArgs {
  Opnd a[2], b[2];  // [0] main segment, [1] LoRA segment (GROUP_M only)
  int K[2];         // GROUP_M: K extent of each segment (K[1] may be 0)
  int M, N;         // GROUP_K: output extent; GROUP_M: N = output columns (features)
  int E;
  const int32_t* offsets;  // [E+1]
  const int4* tiles;       // GROUP_M: {expert, first row, valid rows, -}
  const int32_t* ntiles;   // GROUP_M: number of M tiles (device)
  int ntn;                 // number of N tiles
  int ntm;                 // GROUP_K: number of M tiles
  void* out;
  int64_t out_estride;  // GROUP_K: elements between experts in `out`
  int64_t ld_out;
  void* out2;  // EPI_SWIGLU: act
  int64_t ld_out2;
  const void* aux;  // EPI_SWIGLU_BWD: h
  int64_t ld_aux;
  int I;  // gate width for SwiGLU epilogues / paired weight rows
  float scale;
};

// Spread `total` logical tiles over the 8 XCDs so that each XCD works on a
// contiguous range of them (workgroup b is dispatched to XCD b % 8).
__device__ __forceinline__ int xcd_remap(int b, int total) {
  const int x = b & 7, j = b >> 3, q = total >> 3, rem = total & 7;
  return x * q + (x < rem ? x : rem) + j;
}

// One operand of one tile: where element (mn, k) lives and which ones exist.
template <typename T>
struct View {
  const T* base;
  int64_t ld;
  int kcontig, vec;
  int klim;    // valid k in [0, klim)
  int mn_lim;  // valid local mn in [0, mn_lim) (simple mapping)
  int paired;  // gate_up weight rows: local n < half -> gate row pbase+n, else up row I+pbase+n-half
  int half, pbase, I;
};

template <typename T>
__device__ __forceinline__ int64_t map_mn(const View<T>& v, int n, bool& ok) {
  if (!v.paired) {
    ok = n < v.mn_lim;
    return n;
  }
  const int f = v.pbase + (n < v.half ? n : n - v.half);
  ok = f < v.I;
  return n < v.half ? f : v.I + f;
}

template <typename T>
__device__ __forceinline__ T load_elem(const View<T>& v, int n, int k) {
  bool ok;
  const int64_t g = map_mn(v, n, ok);
  if (!ok || k >= v.klim) return T(0);
  return v.kcontig ? v.base[g * v.ld + k] : v.base[static_cast<int64_t>(k) * v.ld + g];
}

// ----------------------------------------------------------------- epilogue helpers
// Four consecutive columns [col, col+4) of one row; ragged column tails and
// unaligned rows fall back to element stores.
template <typename T>
__device__ __forceinline__ void store4(T* rowp, int col, int ncols, bool aligned,
                                       const float (&v)[4]) {
  if (aligned && col + 4 <= ncols) {
    Vec4<T>::store(rowp + col, v);
  } else {
#pragma unroll
    for (int j = 0; j < 4; ++j)
      if (col + j < ncols) rowp[col + j] = from_f32<T>(v[j]);
  }
}

template <typename T, int MODE, int EPI>
__device__ __forceinline__ void epi_store(const GemmArgs& p, int e, int64_t row0, int m_local,
                                          int rows, int n_col, const float (&v)[4]) {
  if (m_local >= rows) return;
  if (MODE == GROUP_M) {
    const int64_t row = row0 + m_local;
    if (EPI == EPI_STORE) {
      float o[4];
#pragma unroll
      for (int j = 0; j < 4; ++j) o[j] = v[j] * p.scale;
      store4<T>(static_cast<T*>(p.out) + row * p.ld_out, n_col, p.N, (p.ld_out & 3) == 0, o);
    } else if (EPI == EPI_SWIGLU_BWD) {
      if (n_col >= p.N) return;  // N = I (multiple of 8)
      const T* hr = static_cast<const T*>(p.aux) + row * p.ld_aux;
      float g[4], uu[4], dg[4], du[4];
      Vec4<T>::load(hr + n_col, g);
      Vec4<T>::load(hr + p.I + n_col, uu);
#pragma unroll
      for (int j = 0; j < 4; ++j) swiglu_bwd(g[j], uu[j], v[j], dg[j], du[j]);
      T* dr = static_cast<T*>(p.out) + row * p.ld_out;
      Vec4<T>::store(dr + n_col, dg);
      Vec4<T>::store(dr + p.I + n_col, du);
    }
  } else {
    // GROUP_K: out[e][m][n], row = feature m (rows = valid M in this tile)
    float o[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) o[j] = v[j] * p.scale;
    T* rp = static_cast<T*>(p.out) + static_cast<int64_t>(e) * p.out_estride +
            (row0 + m_local) * p.ld_out;
    store4<T>(rp, n_col, p.N, (p.ld_out & 3) == 0, o);
  }
}

template <typename T>
__device__ __forceinline__ void epi_swiglu(const GemmArgs& p, int64_t row0, int m_local,
                                           int rows, int f, const float (&g)[4],
                                           const float (&u)[4]) {
  if (m_local >= rows || f >= p.I) return;  // I multiple of 8: groups of 4 all in or all out
  const int64_t row = row0 + m_local;
  T* hr = static_cast<T*>(p.out) + row * p.ld_out;
  float a[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) a[j] = swiglu(g[j], u[j]);
  Vec4<T>::store(hr + f, g);
  Vec4<T>::store(hr + p.I + f, u);
  Vec4<T>::store(static_cast<T*>(p.out2) + row * p.ld_out2 + f, a);
}

// ----------------------------------------------------------------- bf16 MFMA kernel
// LDS tiles are kBK = 64 deep in k, unpadded, with a 16-byte-chunk XOR swizzle:
//   k-contiguous tile [R][64]: row r keeps k-chunk c at position c ^ (r & 7)
//   n-contiguous tile [64][R]: k-row k keeps n-chunk c at position c ^ nswz<R>(k)
// Fragment reads are bank-conflict free: ds_read_b128 for the first layout,
// ds_read_b64_tr_b16 (CDNA4 LDS transpose read) for the second, and both give
// the same MFMA fragment: lane l holds 8 consecutive k (block l/32) of the
// row or column l%32. Tiles are filled by buffer->LDS DMA (no register
// staging): each wave instruction writes 1 KB of LDS, lane l at +16 l, from a
// per-lane byte offset that encodes the swizzle; lanes outside the operand
// get an out-of-range offset and the hardware writes zeros. Three LDS stages
// keep two tiles in flight while the third is multiplied.
constexpr int kBK = 64;
constexpr int kStages = 3;
constexpr uint32_t kOOB = 0x80000000u;

typedef __attribute__((address_space(3))) void lds_void;
typedef short v4s __attribute__((ext_vector_type(4)));

template <int R>
__device__ __forceinline__ int nswz(int k) {
  return R >= 64 ? ((k & 3) << 1) : 0;
}

template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}

// Own LDS traffic finished, then a workgroup barrier.
__device__ __forceinline__ void barrier_lds() {
  asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

__device__ __forceinline__ int clamp_records(int64_t bytes) {
  return bytes <= 0 ? 0 : (bytes > 0x7fffffff ? 0x7fffffff : static_cast<int>(bytes));
}

// DMA plan of one operand tile: resource, per-instruction lane offsets, k limit.
template <int NI>
struct Plan {
  const void* base;  // buffer resource: base address and size in bytes
  int nrec;
  uint32_t vo[NI];
  int vec;
  int klim;
  int64_t ld;
  View<bf16_t> view;  // element view for the slow (non-DMA) fill
};

// k-contiguous operand of ROWS rows: element (row, k) at base[map(row)*ld + k].
template <int ROWS>
__device__ __forceinline__ void plan_kc(Plan<ROWS / 32>& P, const View<bf16_t>& v,
                                        int64_t bytes, int vec, int wave, int lane) {
  P.view = v;
  P.vec = vec;
  P.klim = v.klim;
  P.ld = v.ld;
  P.base = v.base;
  P.nrec = clamp_records(bytes);
  const int c = (lane & 7) ^ ((lane >> 3) & 7);  // k-chunk this lane fetches
#pragma unroll
  for (int i = 0; i < ROWS / 32; ++i) {
    const int row = 8 * (wave * (ROWS / 32) + i) + (lane >> 3);
    bool ok;
    const int64_t g = map_mn(v, row, ok);
    P.vo[i] = ok ? static_cast<uint32_t>((g * v.ld + c * 8) * 2) : kOOB;
  }
}

// n-contiguous operand of ROWS columns: element (mn, k) at base[k*ld + mn].
template <int ROWS>
__device__ __forceinline__ void plan_nc(Plan<ROWS / 32>& P, const View<bf16_t>& v,
                                        int64_t bytes, int vec, int wave, int lane) {
  P.view = v;
  P.vec = vec;
  P.klim = v.klim;
  P.ld = v.ld;
  P.base = v.base;
  P.nrec = clamp_records(bytes);
  constexpr int CPR = ROWS / 8;        // 16-byte chunks per k-row
  constexpr int KPI = 64 / CPR;        // k-rows per 1 KB instruction
#pragma unroll
  for (int i = 0; i < ROWS / 32; ++i) {
    const int kr = (wave * (ROWS / 32) + i) * KPI + lane / CPR;
    const int cn = (lane % CPR) ^ nswz<ROWS>(kr);
    P.vo[i] = cn * 8 < v.mn_lim ? static_cast<uint32_t>((kr * v.ld + cn * 8) * 2) : kOOB;
  }
}

// Issue one tile: DMA when possible, else an element-wise fill.
template <int ROWS, bool KC>
__device__ __forceinline__ void fill(const Plan<ROWS / 32>& P, int k0, char* lds, int wave,
                                     int lane) {
  if (P.vec) {
    uint32_t soff;
    bool tail = false;
    if (KC) {
      soff = static_cast<uint32_t>(k0) * 2;
      tail = k0 + kBK > P.klim;
    } else {
      soff = static_cast<uint32_t>(k0 * P.ld * 2);
    }
    const int kc = ((lane & 7) ^ ((lane >> 3) & 7)) * 8;
    const bool kok = !tail || (k0 + kc < P.klim);
    const __amdgpu_buffer_rsrc_t rs =
        __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(P.base), 0, P.nrec, 0x00020000);
#pragma unroll
    for (int i = 0; i < ROWS / 32; ++i) {
      const uint32_t vo = kok ? P.vo[i] : kOOB;
      __builtin_amdgcn_raw_ptr_buffer_load_lds(
          rs, (lds_void*)(lds + (wave * (ROWS / 32) + i) * 1024), 16, vo, soff, 0, 0);
    }
  } else {
    bf16_t* t = reinterpret_cast<bf16_t*>(lds);
    for (int e = threadIdx.x; e < ROWS * kBK; e += 256) {
      int byte;
      bf16_t val;
      if (KC) {
        const int row = e / kBK, k = e % kBK;
        byte = row * 128 + ((((k >> 3) ^ (row & 7))) << 4) + (k & 7) * 2;
        val = load_elem(P.view, row, k0 + k);
      } else {
        const int k = e / ROWS, mn = e % ROWS;
        byte = k * ROWS * 2 + (((mn >> 3) ^ nswz<ROWS>(k)) << 4) + (mn & 7) * 2;
        val = load_elem(P.view, mn, k0 + k);
      }
      t[byte >> 1] = val;
    }
  }
}

// Per-lane LDS byte offsets of the MFMA fragments.
template <int ROWS, bool KC, int NFR>
struct FragAddr {
  int off[KC ? 4 : NFR];  // KC: per k-step (same for all fragments); NC: per fragment
};

template <int ROWS, bool KC, int NFR>
__device__ __forceinline__ void frag_addr(FragAddr<ROWS, KC, NFR>& F, const int (&fr_base)[NFR],
                                          int lane) {
  if (KC) {
    const int h = lane >> 5;
#pragma unroll
    for (int ks = 0; ks < 4; ++ks)
      F.off[ks] = (lane & 31) * 128 + ((((2 * ks + h) ^ (lane & 7))) << 4);
  } else {
    const int G = lane >> 4, li = lane & 15;
    const int kl = (G >> 1) * 8 + (li >> 2);  // k row of this lane within a k-step (call 0)
#pragma unroll
    for (int f = 0; f < (KC ? 0 : NFR); ++f) {
      const int n = fr_base[f] + (G & 1) * 16 + (li & 3) * 4;
      F.off[KC ? 0 : f] = kl * ROWS * 2 + ((((n >> 3) ^ nswz<ROWS>(kl))) << 4) + (n & 7) * 2;
    }
  }
}

template <int ROWS, bool KC, int NFR>
__device__ __forceinline__ bf16x8 read_frag(const char* tile, const FragAddr<ROWS, KC, NFR>& F,
                                            int f, int fr_base_f, int ks) {
  if (KC) {
    return *reinterpret_cast<const bf16x8*>(tile + fr_base_f * 128 + F.off[ks]);
  } else {
    const char* p = tile + F.off[KC ? 0 : f] + ks * 16 * ROWS * 2;
    v4s lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) v4s*)(p));
    v4s hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
        (__attribute__((address_space(3))) v4s*)(p + 4 * ROWS * 2));
    typedef short v8s __attribute__((ext_vector_type(8)));
    v8s r = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
    return __builtin_bit_cast(bf16x8, r);
  }
}

template <int BM, int BN, int WM, int WN, int MODE, int EPI, bool PAIRED, bool A_KC, bool B_KC>
__global__ __launch_bounds__(256) void gemm_bf16(GemmArgs p) {
  constexpr int WAVES_N = BN / WN, MF = WM / 32, NF = WN / 32;
  constexpr int A_BYTES = BM * kBK * 2, B_BYTES = BN * kBK * 2, ST = A_BYTES + B_BYTES;
  constexpr int NIA = BM / 32, NIB = BN / 32;  // DMA instructions per wave per stage
  static_assert((BM / WM) * (BN / WN) == 4, "four waves per block");
  static_assert(!PAIRED || (NF % 2 == 0), "paired tiles need gate and up fragments");
  __shared__ __attribute__((aligned(1024))) char smem[kStages * ST];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave / WAVES_N, wn = wave % WAVES_N;

  int e, n_tile, rows, m0 = 0, krows = 0;
  int64_t row0;
  if (MODE == GROUP_M) {
    const int mtot = *p.ntiles;
    const int total = mtot * p.ntn;
    if (static_cast<int>(blockIdx.x) >= total) return;
    // XCD-contiguous ranges, then groups of 8 M tiles swept across all N tiles,
    // so the tiles an XCD runs together share A rows and weight columns in L2.
    const int L = xcd_remap(blockIdx.x, total);
    constexpr int GM = 8;
    const int mg = L / (GM * p.ntn);
    const int gbase = mg * GM;
    const int gsz = min(GM, mtot - gbase);
    const int rem = L - gbase * p.ntn;
    n_tile = rem / gsz;
    const int mt = gbase + rem % gsz;
    const int4 t = p.tiles[mt];
    e = t.x;
    row0 = t.y;
    rows = t.z;
  } else {
    const int total = p.E * p.ntm * p.ntn;
    if (static_cast<int>(blockIdx.x) >= total) return;
    const int L = xcd_remap(blockIdx.x, total);
    e = L / (p.ntm * p.ntn);
    const int rem = L - e * (p.ntm * p.ntn);
    const int mt = rem / p.ntn;
    n_tile = rem - mt * p.ntn;
    m0 = mt * BM;
    rows = min(BM, p.M - m0);
    row0 = p.offsets[e];
    krows = p.offsets[e + 1] - static_cast<int>(row0);
  }
  const int n0 = PAIRED ? 0 : n_tile * BN;

  // ---- DMA plans for the main segment (0) and the LoRA segment (1)
  Plan<NIA> pa[2];
  Plan<NIB> pb[2];
  const int nseg = MODE == GROUP_M ? 2 : 1;
#pragma unroll
  for (int seg = 0; seg < 2; ++seg) {
    if (seg >= nseg) break;
    const Opnd& A = p.a[seg];
    const Opnd& B = p.b[seg];
    View<bf16_t> va{}, vb{};
    va.ld = A.ld; va.kcontig = A.kcontig; va.vec = A.vec;
    vb.ld = B.ld; vb.kcontig = B.kcontig; vb.vec = B.vec;
    int64_t abytes, bbytes;
    if (MODE == GROUP_M) {
      const int K = p.K[seg];
      va.base = static_cast<const bf16_t*>(A.ptr) + row0 * A.ld;
      va.klim = K;
      va.mn_lim = rows;
      abytes = static_cast<int64_t>(rows) * A.ld * 2;
      const bf16_t* wb = static_cast<const bf16_t*>(B.ptr) + static_cast<int64_t>(e) * B.estride;
      vb.klim = K;
      if (PAIRED) {
        vb.base = wb;
        vb.paired = 1;
        vb.half = BN / 2;
        vb.pbase = n_tile * (BN / 2);
        vb.I = p.I;
        vb.mn_lim = BN;
        bbytes = static_cast<int64_t>(2) * p.I * B.ld * 2;
      } else if (B_KC) {
        vb.base = wb + static_cast<int64_t>(n0) * B.ld;
        vb.mn_lim = p.N - n0;
        bbytes = static_cast<int64_t>(p.N - n0) * B.ld * 2;
      } else {
        vb.base = wb + n0;
        vb.mn_lim = p.N - n0;
        bbytes = static_cast<int64_t>(K) * B.ld * 2 - static_cast<int64_t>(n0) * 2;
      }
    } else {
      va.base = static_cast<const bf16_t*>(A.ptr) + row0 * A.ld + m0;
      va.klim = krows;
      va.mn_lim = p.M - m0;
      abytes = static_cast<int64_t>(krows) * A.ld * 2 - static_cast<int64_t>(m0) * 2;
      vb.base = static_cast<const bf16_t*>(B.ptr) + row0 * B.ld + n0;
      vb.klim = krows;
      vb.mn_lim = p.N - n0;
      bbytes = static_cast<int64_t>(krows) * B.ld * 2 - static_cast<int64_t>(n0) * 2;
    }
    if (A_KC) plan_kc<BM>(pa[seg], va, abytes, A.vec, wave, lane);
    else plan_nc<BM>(pa[seg], va, abytes, A.vec, wave, lane);
    if (B_KC) plan_kc<BN>(pb[seg], vb, bbytes, B.vec, wave, lane);
    else plan_nc<BN>(pb[seg], vb, bbytes, B.vec, wave, lane);
  }

  const int nk0 = MODE == GROUP_M ? (p.K[0] + kBK - 1) / kBK : (krows + kBK - 1) / kBK;
  const int nk1 = MODE == GROUP_M ? (p.K[1] + kBK - 1) / kBK : 0;
  const int nk = nk0 + nk1;

  auto issue = [&](int j) {
    char* sa = smem + (j % kStages) * ST;
    char* sb = sa + A_BYTES;
    if (j < nk0) {
      fill<BM, A_KC>(pa[0], j * kBK, sa, wave, lane);
      fill<BN, B_KC>(pb[0], j * kBK, sb, wave, lane);
    } else {
      fill<BM, A_KC>(pa[1], (j - nk0) * kBK, sa, wave, lane);
      fill<BN, B_KC>(pb[1], (j - nk0) * kBK, sb, wave, lane);
    }
  };
  // DMA-only stage: the number of loads it leaves outstanding is known.
  auto dma_stage = [&](int j) { return j < nk0 ? (pa[0].vec && pb[0].vec) : (pa[1].vec && pb[1].vec); };

  // fragment row bases (in tile rows) and lane offsets
  int fa_base[MF], fb_base[NF];
#pragma unroll
  for (int mi = 0; mi < MF; ++mi) fa_base[mi] = wm * WM + mi * 32;
#pragma unroll
  for (int ni = 0; ni < NF; ++ni) {
    if (PAIRED)
      fb_base[ni] = (ni < NF / 2) ? wn * (WN / 2) + ni * 32 : BN / 2 + wn * (WN / 2) + (ni - NF / 2) * 32;
    else
      fb_base[ni] = wn * WN + ni * 32;
  }
  FragAddr<BM, A_KC, MF> FA;
  FragAddr<BN, B_KC, NF> FB;
  frag_addr<BM, A_KC, MF>(FA, fa_base, lane);
  frag_addr<BN, B_KC, NF>(FB, fb_base, lane);

  f32x16 acc[MF][NF];
#pragma unroll
  for (int i = 0; i < MF; ++i)
#pragma unroll
    for (int j = 0; j < NF; ++j)
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[i][j][v] = 0.f;

  if (nk > 0) issue(0);
  if (nk > 1) issue(1);
  for (int it = 0; it < nk; ++it) {
    if (it + 1 < nk && dma_stage(it + 1))
      wait_vmcnt<NIA + NIB>();
    else
      wait_vmcnt<0>();
    barrier_lds();
    if (it + 2 < nk) issue(it + 2);
    const char* sa = smem + (it % kStages) * ST;
    const char* sb = sa + A_BYTES;
#pragma unroll
    for (int ks = 0; ks < kBK / 16; ++ks) {
      bf16x8 af[MF], bf[NF];
#pragma unroll
      for (int mi = 0; mi < MF; ++mi) af[mi] = read_frag<BM, A_KC, MF>(sa, FA, mi, fa_base[mi], ks);
#pragma unroll
      for (int ni = 0; ni < NF; ++ni) bf[ni] = read_frag<BN, B_KC, NF>(sb, FB, ni, fb_base[ni], ks);
#pragma unroll
      for (int mi = 0; mi < MF; ++mi)
#pragma unroll
        for (int ni = 0; ni < NF; ++ni)
          acc[mi][ni] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(bf[ni], af[mi], acc[mi][ni], 0, 0, 0);
    }
  }

  // Lane holds, for MFMA tile (mi, ni), row m = wm*WM + mi*32 + lane%32 and the
  // columns 8*(v/4) + 4*(lane/32) + v%4 of the tile's 32 weight rows.
  const int m_lane = wm * WM + (lane & 31);
  const int c_lane = 4 * (lane >> 5);
  if (PAIRED) {
#pragma unroll
    for (int mi = 0; mi < MF; ++mi)
#pragma unroll
      for (int ni = 0; ni < NF / 2; ++ni)
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          float g[4], u[4];
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            g[j] = acc[mi][ni][4 * q + j];
            u[j] = acc[mi][ni + NF / 2][4 * q + j];
          }
          const int f = n_tile * (BN / 2) + wn * (WN / 2) + ni * 32 + 8 * q + c_lane;
          epi_swiglu<bf16_t>(p, row0, m_lane + mi * 32, rows, f, g, u);
        }
  } else {
    const int64_t rbase = MODE == GROUP_M ? row0 : static_cast<int64_t>(m0);
#pragma unroll
    for (int mi = 0; mi < MF; ++mi)
#pragma unroll
      for (int ni = 0; ni < NF; ++ni)
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          float v[4];
#pragma unroll
          for (int j = 0; j < 4; ++j) v[j] = acc[mi][ni][4 * q + j];
          const int col = n0 + wn * WN + ni * 32 + 8 * q + c_lane;
          epi_store<bf16_t, MODE, EPI>(p, e, rbase, m_lane + mi * 32, rows, col, v);
        }
  }
}

// ----------------------------------------------------------------- float32 FMA kernel
// 64 x 64 tiles (paired: 64 gate + 64 up columns), 4 x 4 outputs per thread.
template <int MODE, int EPI, bool PAIRED>
__global__ __launch_bounds__(256) void gemm_f32(GemmArgs p) {
  constexpr int BM = 64, BN = 64, BK = 16, NB = PAIRED ? 2 * BN : BN;
  __shared__ float sA[BK][BM + 4];
  __shared__ float sB[BK][NB + 4];
  const int tid = threadIdx.x, tx = tid & 15, ty = tid >> 4;

  int e, n_tile, rows, m0 = 0, krows = 0;
  int64_t row0;
  if (MODE == GROUP_M) {
    const int mtot = *p.ntiles;
    const int total = mtot * p.ntn;
    if (static_cast<int>(blockIdx.x) >= total) return;
    const int mt = blockIdx.x % mtot;
    n_tile = blockIdx.x / mtot;
    const int4 t = p.tiles[mt];
    e = t.x;
    row0 = t.y;
    rows = t.z;
  } else {
    const int total = p.E * p.ntm * p.ntn;
    if (static_cast<int>(blockIdx.x) >= total) return;
    e = blockIdx.x / (p.ntm * p.ntn);
    const int rem = blockIdx.x - e * (p.ntm * p.ntn);
    const int mt = rem / p.ntn;
    n_tile = rem - mt * p.ntn;
    m0 = mt * BM;
    rows = min(BM, p.M - m0);
    row0 = p.offsets[e];
    krows = p.offsets[e + 1] - static_cast<int>(row0);
  }
  const int n0 = PAIRED ? 0 : n_tile * BN;

  float acc[4][4] = {}, accu[4][4] = {};
  const int nseg = MODE == GROUP_M ? 2 : 1;
  for (int seg = 0; seg < nseg; ++seg) {
    const Opnd& A = p.a[seg];
    const Opnd& B = p.b[seg];
    View<float> va{}, vb{};
    va.ld = A.ld; va.kcontig = A.kcontig; vb.ld = B.ld; vb.kcontig = B.kcontig;
    int K;
    if (MODE == GROUP_M) {
      K = p.K[seg];
      va.base = static_cast<const float*>(A.ptr) + row0 * A.ld;
      va.mn_lim = rows;
      const float* wb = static_cast<const float*>(B.ptr) + static_cast<int64_t>(e) * B.estride;
      if (PAIRED) {
        vb.base = wb; vb.paired = 1; vb.half = BN; vb.pbase = n_tile * BN; vb.I = p.I;
        vb.mn_lim = NB;
      } else {
        vb.base = B.kcontig ? wb + static_cast<int64_t>(n0) * B.ld : wb + n0;
        vb.mn_lim = p.N - n0;
      }
    } else {
      K = krows;
      va.base = static_cast<const float*>(A.ptr) + row0 * A.ld + m0;
      va.mn_lim = p.M - m0;
      vb.base = static_cast<const float*>(B.ptr) + row0 * B.ld + n0;
      vb.mn_lim = p.N - n0;
    }
    va.klim = K;
    vb.klim = K;
    for (int k0 = 0; k0 < K; k0 += BK) {
      for (int i = tid; i < BM * BK; i += 256) sA[i % BK][i / BK] = load_elem(va, i / BK, k0 + i % BK);
      for (int i = tid; i < NB * BK; i += 256) sB[i % BK][i / BK] = load_elem(vb, i / BK, k0 + i % BK);
      __syncthreads();
#pragma unroll
      for (int kk = 0; kk < BK; ++kk) {
        float a[4], b[4], bu[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) a[i] = sA[kk][ty * 4 + i];
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          b[j] = sB[kk][tx * 4 + j];
          bu[j] = PAIRED ? sB[kk][BN + tx * 4 + j] : 0.f;
        }
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            acc[i][j] = fmaf(a[i], b[j], acc[i][j]);
            if (PAIRED) accu[i][j] = fmaf(a[i], bu[j], accu[i][j]);
          }
      }
      __syncthreads();
    }
  }
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    float v[4], u[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      v[j] = acc[i][j];
      u[j] = accu[i][j];
    }
    if (PAIRED) {
      epi_swiglu<float>(p, row0, ty * 4 + i, rows, n_tile * BN + tx * 4, v, u);
    } else {
      const int64_t rbase = MODE == GROUP_M ? row0 : static_cast<int64_t>(m0);
      epi_store<float, MODE, EPI>(p, e, rbase, ty * 4 + i, rows, n0 + tx * 4, v);
    }
  }
}

// ----------------------------------------------------------------- tile list
// One block of 1024 threads (E <= 1024): M tiles of `bm` rows per expert, in
// expert order; empty experts get none.
__global__ __launch_bounds__(1024) void tiles_kernel(const int32_t* __restrict__ offsets, int E,
                                                     int bm, int4* __restrict__ tiles,
                                                     int32_t* __restrict__ ntiles) {
  __shared__ int wsum[1024 / kWave];
  const int lane = threadIdx.x & (kWave - 1), wave = threadIdx.x / kWave;
  const int e = threadIdx.x;
  int lo = 0, cnt = 0;
  if (e < E) {
    lo = offsets[e];
    cnt = offsets[e + 1] - lo;
  }
  const int nt = (cnt + bm - 1) / bm;
  int incl = nt;
#pragma unroll
  for (int off = 1; off < kWave; off <<= 1) {
    int o = __shfl_up(incl, off, kWave);
    if (lane >= off) incl += o;
  }
  if (lane == kWave - 1) wsum[wave] = incl;
  __syncthreads();
  int base = 0, total = 0;
  for (int w = 0; w < 1024 / kWave; ++w) {
    if (w < wave) base += wsum[w];
    total += wsum[w];
  }
  base += incl - nt;
  for (int i = 0; i < nt; ++i) {
    const int r = i * bm;
    tiles[base + i] = make_int4(e, lo + r, min(bm, cnt - r), 0);
  }
  if (threadIdx.x == 0) *ntiles = total;
}

// ----------------------------------------------------------------- host side
constexpr size_t kAlign = 256;
inline size_t align_up(size_t x) { return (x + kAlign - 1) / kAlign * kAlign; }

inline int ceil_div(int64_t a, int64_t b) { return static_cast<int>((a + b - 1) / b); }

inline bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15) == 0; }

Opnd opnd(const void* ptr, int64_t estride, int64_t ld, int kcontig, bool vec_ok) {
  Opnd o;
  o.ptr = ptr;
  o.estride = estride;
  o.ld = ld;
  o.kcontig = kcontig;
  o.vec = vec_ok && (ld % 8 == 0) && aligned16(ptr) && (estride % 8 == 0);
  return o;
}

Opnd none() { return Opnd{nullptr, 0, 0, 1, 0}; }

// Tile list capacity for `bm`-row tiles.
inline int64_t tile_cap(int64_t N, int E, int bm) { return (N + bm - 1) / bm + E + 1; }

struct WsLayout {
  int4* tiles;
  int32_t* ntiles;
  size_t bytes;
};

inline int tile_rows(int dtype) { return dtype == MOE_BF16 ? 128 : 64; }

WsLayout tile_ws(void* ws, const ExpertDims& d) {
  WsLayout L;
  const int bm = tile_rows(d.dtype);
  const size_t tb = align_up(static_cast<size_t>(tile_cap(d.N, d.E, bm)) * sizeof(int4));
  L.tiles = static_cast<int4*>(ws);
  L.ntiles = reinterpret_cast<int32_t*>(static_cast<char*>(ws) + tb);
  L.bytes = tb + kAlign;
  return L;
}

template <typename K>
hipError_t launch(K kern, int grid, const GemmArgs& a, hipStream_t s) {
  if (grid <= 0) return hipSuccess;
  hipLaunchKernelGGL(kern, dim3(grid), dim3(256), 0, s, a);
  return hipGetLastError();
}

// M-tile grid bound for GROUP_M launches (excess blocks exit at once).
inline int gm_grid(const ExpertDims& d, int ntn) {
  return static_cast<int>(tile_cap(d.N, d.E, tile_rows(d.dtype)) * ntn);
}

GemmArgs base_args(const ExpertDims& d, const int32_t* offsets, const WsLayout& L) {
  GemmArgs a{};
  a.a[1] = none();
  a.b[1] = none();
  a.E = d.E;
  a.offsets = offsets;
  a.tiles = L.tiles;
  a.ntiles = L.ntiles;
  a.I = d.I;
  a.scale = 1.0f;
  return a;
}

// out[rows, r] = scale * A[rows, K] * L_e (L_e is [r, K] when l_kcontig, else [K, r]).
hipError_t side_product(const ExpertDims& d, const int32_t* offsets, const WsLayout& L,
                        const void* A, int K, const void* Lw, int64_t l_estride, int l_kcontig,
                        void* out, hipStream_t s) {
  GemmArgs a = base_args(d, offsets, L);
  const bool r_vec = d.r % 8 == 0;
  a.a[0] = opnd(A, 0, K, 1, true);
  a.b[0] = l_kcontig ? opnd(Lw, l_estride, K, 1, true) : opnd(Lw, l_estride, d.r, 0, r_vec);
  a.K[0] = K;
  a.K[1] = 0;
  a.N = d.r;
  a.out = out;
  a.ld_out = d.r;
  a.scale = d.scale;
  if (d.dtype == MOE_BF16) {
    a.ntn = 1;
    if (l_kcontig) {
      if (d.r <= 32)
        return launch(gemm_bf16<128, 32, 32, 32, GROUP_M, EPI_STORE, false, true, true>,
                      gm_grid(d, 1), a, s);
      return launch(gemm_bf16<128, 64, 32, 64, GROUP_M, EPI_STORE, false, true, true>,
                    gm_grid(d, 1), a, s);
    }
    if (d.r <= 32)
      return launch(gemm_bf16<128, 32, 32, 32, GROUP_M, EPI_STORE, false, true, false>,
                    gm_grid(d, 1), a, s);
    return launch(gemm_bf16<128, 64, 32, 64, GROUP_M, EPI_STORE, false, true, false>,
                  gm_grid(d, 1), a, s);
  }
  a.ntn = ceil_div(d.r, 64);
  return launch(gemm_f32<GROUP_M, EPI_STORE, false>, gm_grid(d, a.ntn), a, s);
}

// out_e[P, Q] = sum over the expert's rows n of L[n, P] R[n, Q]  (L: [rows, P], R: [rows, Q]).
hipError_t weight_grad(const ExpertDims& d, const int32_t* offsets, const void* Lm, int P,
                       const void* Rm, int Q, void* out, hipStream_t s) {
  GemmArgs a{};
  a.a[1] = none();
  a.b[1] = none();
  a.E = d.E;
  a.offsets = offsets;
  a.M = P;
  a.N = Q;
  a.scale = 1.0f;
  a.out = out;
  a.out_estride = static_cast<int64_t>(P) * Q;
  a.ld_out = Q;
  a.a[0] = opnd(Lm, 0, P, 0, P % 8 == 0);
  a.b[0] = opnd(Rm, 0, Q, 0, Q % 8 == 0);
  if (d.dtype == MOE_BF16) {
    if (Q <= 64 && P > 64) {  // [big, r]
      a.ntn = 1;
      if (Q <= 32) {
        a.ntm = ceil_div(P, 256);
        return launch(gemm_bf16<256, 32, 64, 32, GROUP_K, EPI_STORE, false, false, false>, d.E * a.ntm, a, s);
      }
      a.ntm = ceil_div(P, 256);
      return launch(gemm_bf16<256, 64, 64, 64, GROUP_K, EPI_STORE, false, false, false>, d.E * a.ntm, a, s);
    }
    // [r, big] (or both small)
    a.ntn = ceil_div(Q, 256);
    if (P <= 32) {
      a.ntm = 1;
      return launch(gemm_bf16<32, 256, 32, 64, GROUP_K, EPI_STORE, false, false, false>, d.E * a.ntn, a, s);
    }
    a.ntm = ceil_div(P, 64);
    return launch(gemm_bf16<64, 256, 64, 64, GROUP_K, EPI_STORE, false, false, false>, d.E * a.ntm * a.ntn, a,
                  s);
  }
  a.ntm = ceil_div(P, 64);
  a.ntn = ceil_div(Q, 64);
  return launch(gemm_f32<GROUP_K, EPI_STORE, false>, d.E * a.ntm * a.ntn, a, s);
}

#define MOE_TRY(x)                      \
  do {                                  \
    hipError_t err_ = (x);              \
    if (err_ != hipSuccess) return err_; \
  } while (0)

}  // namespace

size_t experts_fwd_ws_bytes(const ExpertDims& d) {
  return tile_ws(nullptr, d).bytes;
}

size_t experts_bwd_ws_bytes(const ExpertDims& d) {
  const size_t esz = d.dtype == MOE_BF16 ? 2 : 4;
  size_t b = tile_ws(nullptr, d).bytes;
  b += align_up(static_cast<size_t>(d.N) * d.r * esz) * 2;        // G B_d, dH B_gu
  b += align_up(static_cast<size_t>(d.N) * 2 * d.I * esz);         // dH
  return b;
}

hipError_t launch_experts_fwd(const ExpertDims& d, const void* x_perm, const int32_t* offsets,
                              const moe_weights& w, const moe_saved& sv, void* ws,
                              hipStream_t s, KernelTimer* tm) {
  const WsLayout L = tile_ws(ws, d);
  const int bm = tile_rows(d.dtype);
  const int H = d.H, I = d.I, r = d.r;
  hipLaunchKernelGGL(tiles_kernel, dim3(1), dim3(1024), 0, s, offsets, d.E, bm, L.tiles,
                     L.ntiles);
  MOE_TRY(hipGetLastError());
  {  // u_gu = s X A_gu^T
    TimedScope ts(tm, MOE_K_LORA_SIDE, s);
    MOE_TRY(side_product(d, offsets, L, x_perm, H, w.a_gu, static_cast<int64_t>(r) * H, 1,
                         sv.u_gu, s));
  }
  {  // h = X W_gu^T + u_gu B_gu^T ; act = SwiGLU(h)
    GemmArgs a = base_args(d, offsets, L);
    a.a[0] = opnd(x_perm, 0, H, 1, true);
    a.b[0] = opnd(w.w_gu, static_cast<int64_t>(2) * I * H, H, 1, true);
    a.a[1] = opnd(sv.u_gu, 0, r, 1, r % 8 == 0);
    a.b[1] = opnd(w.b_gu, static_cast<int64_t>(2) * I * r, r, 1, r % 8 == 0);
    a.K[0] = H;
    a.K[1] = r;
    a.N = 2 * I;
    a.out = sv.h;
    a.ld_out = 2 * I;
    a.out2 = sv.act;
    a.ld_out2 = I;
    TimedScope ts(tm, MOE_K_GATE_UP_FWD, s);
    if (d.dtype == MOE_BF16) {
      a.ntn = ceil_div(I, 128);
      MOE_TRY(launch(gemm_bf16<128, 256, 64, 128, GROUP_M, EPI_SWIGLU, true, true, true>, gm_grid(d, a.ntn),
                     a, s));
    } else {
      a.ntn = ceil_div(I, 64);
      MOE_TRY(launch(gemm_f32<GROUP_M, EPI_SWIGLU, true>, gm_grid(d, a.ntn), a, s));
    }
  }
  {  // u_d = s act A_d^T
    TimedScope ts(tm, MOE_K_LORA_SIDE, s);
    MOE_TRY(side_product(d, offsets, L, sv.act, I, w.a_d, static_cast<int64_t>(r) * I, 1,
                         sv.u_d, s));
  }
  {  // y_exp = act W_d^T + u_d B_d^T
    GemmArgs a = base_args(d, offsets, L);
    a.a[0] = opnd(sv.act, 0, I, 1, true);
    a.b[0] = opnd(w.w_d, static_cast<int64_t>(H) * I, I, 1, true);
    a.a[1] = opnd(sv.u_d, 0, r, 1, r % 8 == 0);
    a.b[1] = opnd(w.b_d, static_cast<int64_t>(H) * r, r, 1, r % 8 == 0);
    a.K[0] = I;
    a.K[1] = r;
    a.N = H;
    a.out = sv.y_exp;
    a.ld_out = H;
    TimedScope ts(tm, MOE_K_DOWN_FWD, s);
    if (d.dtype == MOE_BF16) {
      a.ntn = ceil_div(H, 256);
      MOE_TRY(launch(gemm_bf16<128, 256, 64, 128, GROUP_M, EPI_STORE, false, true, true>, gm_grid(d, a.ntn),
                     a, s));
    } else {
      a.ntn = ceil_div(H, 64);
      MOE_TRY(launch(gemm_f32<GROUP_M, EPI_STORE, false>, gm_grid(d, a.ntn), a, s));
    }
  }
  return hipSuccess;
}

hipError_t launch_experts_bwd(const ExpertDims& d, const void* g, const void* x_perm,
                              const int32_t* offsets, const moe_weights& w,
                              const moe_saved& sv, void* dx_perm, const moe_lora_grads& gr,
                              void* ws, hipStream_t s, KernelTimer* tm) {
  const WsLayout L = tile_ws(ws, d);
  const int bm = tile_rows(d.dtype);
  const int H = d.H, I = d.I, r = d.r;
  const size_t esz = d.dtype == MOE_BF16 ? 2 : 4;
  char* p = static_cast<char*>(ws) + L.bytes;
  void* gb = p;
  p += align_up(static_cast<size_t>(d.N) * r * esz);
  void* dhb = p;
  p += align_up(static_cast<size_t>(d.N) * r * esz);
  void* dh = p;

  hipLaunchKernelGGL(tiles_kernel, dim3(1), dim3(1024), 0, s, offsets, d.E, bm, L.tiles,
                     L.ntiles);
  MOE_TRY(hipGetLastError());
  {  // gb = s G B_d      (B_d[e] is [H, r]: K = H rows, r contiguous)
    TimedScope ts(tm, MOE_K_LORA_SIDE, s);
    MOE_TRY(side_product(d, offsets, L, g, H, w.b_d, static_cast<int64_t>(H) * r, 0, gb, s));
  }
  {  // dAct = G W_d + gb A_d ; dH = SwiGLU'(h) dAct
    GemmArgs a = base_args(d, offsets, L);
    a.a[0] = opnd(g, 0, H, 1, true);
    a.b[0] = opnd(w.w_d, static_cast<int64_t>(H) * I, I, 0, true);   // [K=H][N=I]
    a.a[1] = opnd(gb, 0, r, 1, r % 8 == 0);
    a.b[1] = opnd(w.a_d, static_cast<int64_t>(r) * I, I, 0, true);   // [K=r][N=I]
    a.K[0] = H;
    a.K[1] = r;
    a.N = I;
    a.out = dh;
    a.ld_out = 2 * I;
    a.aux = sv.h;
    a.ld_aux = 2 * I;
    TimedScope ts(tm, MOE_K_DOWN_BWD, s);
    if (d.dtype == MOE_BF16) {
      a.ntn = ceil_div(I, 256);
      MOE_TRY(launch(gemm_bf16<128, 256, 64, 128, GROUP_M, EPI_SWIGLU_BWD, false, true, false>,
                     gm_grid(d, a.ntn), a, s));
    } else {
      a.ntn = ceil_div(I, 64);
      MOE_TRY(launch(gemm_f32<GROUP_M, EPI_SWIGLU_BWD, false>, gm_grid(d, a.ntn), a, s));
    }
  }
  {  // dB_d = G^T u_d  [H, r] ;  dA_d = gb^T act  [r, I]
    TimedScope ts(tm, MOE_K_LORA_WGRAD, s);
    MOE_TRY(weight_grad(d, offsets, g, H, sv.u_d, r, gr.db_d, s));
    MOE_TRY(weight_grad(d, offsets, gb, r, sv.act, I, gr.da_d, s));
  }
  {  // dhb = s dH B_gu   (B_gu[e] is [2I, r])
    TimedScope ts(tm, MOE_K_LORA_SIDE, s);
    MOE_TRY(side_product(d, offsets, L, dh, 2 * I, w.b_gu, static_cast<int64_t>(2) * I * r, 0,
                         dhb, s));
  }
  {  // dX = dH W_gu + dhb A_gu
    GemmArgs a = base_args(d, offsets, L);
    a.a[0] = opnd(dh, 0, 2 * I, 1, true);
    a.b[0] = opnd(w.w_gu, static_cast<int64_t>(2) * I * H, H, 0, true);  // [K=2I][N=H]
    a.a[1] = opnd(dhb, 0, r, 1, r % 8 == 0);
    a.b[1] = opnd(w.a_gu, static_cast<int64_t>(r) * H, H, 0, true);      // [K=r][N=H]
    a.K[0] = 2 * I;
    a.K[1] = r;
    a.N = H;
    a.out = dx_perm;
    a.ld_out = H;
    TimedScope ts(tm, MOE_K_GATE_UP_BWD, s);
    if (d.dtype == MOE_BF16) {
      a.ntn = ceil_div(H, 256);
      MOE_TRY(launch(gemm_bf16<128, 256, 64, 128, GROUP_M, EPI_STORE, false, true, false>, gm_grid(d, a.ntn),
                     a, s));
    } else {
      a.ntn = ceil_div(H, 64);
      MOE_TRY(launch(gemm_f32<GROUP_M, EPI_STORE, false>, gm_grid(d, a.ntn), a, s));
    }
  }
  {  // dB_gu = dH^T u_gu  [2I, r] ;  dA_gu = dhb^T X  [r, H]
    TimedScope ts(tm, MOE_K_LORA_WGRAD, s);
    MOE_TRY(weight_grad(d, offsets, dh, 2 * I, sv.u_gu, r, gr.db_gu, s));
    MOE_TRY(weight_grad(d, offsets, dhb, r, x_perm, H, gr.da_gu, s));
  }
  return hipSuccess;
}

}  // namespace moe
