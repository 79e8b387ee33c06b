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

// ----------------------------------------------------------------- tile staging (bf16)
template <int ROWS, int BK>
struct Regs {
  static constexpr int CPR = BK / 8;               // 16-byte chunks per row (k contiguous)
  static constexpr int CH = ROWS * CPR;            // chunks per tile
  static constexpr int PER_K = (CH + 255) / 256;   // chunks per thread, k-contiguous
  static constexpr int NBLK = ROWS * BK / 32;      // 4(k) x 8(mn) blocks, transposed
  static constexpr int PER_B = (NBLK + 255) / 256;
  static constexpr int NR = PER_K > 4 * PER_B ? PER_K : 4 * PER_B;
  uint4 r[NR];
};

// Global -> registers (vector modes only; the scalar mode loads in commit()).
template <int ROWS, int BK>
__device__ __forceinline__ void fetch(const View<bf16_t>& v, int k0, Regs<ROWS, BK>& R) {
  typedef Regs<ROWS, BK> RG;
  const int tid = threadIdx.x;
  if (!v.vec) return;
  if (v.kcontig) {
#pragma unroll
    for (int i = 0; i < RG::PER_K; ++i) {
      const int c = tid + 256 * i;
      const int row = c / RG::CPR, kc = c % RG::CPR;
      uint4 val = make_uint4(0, 0, 0, 0);
      if (c < RG::CH) {
        bool ok;
        const int64_t g = map_mn(v, row, ok);
        const int k = k0 + kc * 8;
        if (ok && k < v.klim) val = *reinterpret_cast<const uint4*>(v.base + g * v.ld + k);
      }
      R.r[i] = val;
    }
  } else {
    constexpr int MNC = ROWS / 8;
#pragma unroll
    for (int i = 0; i < RG::PER_B; ++i) {
      const int b = tid + 256 * i;
      const int mnc = b % MNC, kq = b / MNC;
      const bool ok = b < RG::NBLK && mnc * 8 < v.mn_lim;
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int k = k0 + kq * 4 + q;
        uint4 val = make_uint4(0, 0, 0, 0);
        if (ok && k < v.klim)
          val = *reinterpret_cast<const uint4*>(v.base + static_cast<int64_t>(k) * v.ld + mnc * 8);
        R.r[4 * i + q] = val;
      }
    }
  }
}

__device__ __forceinline__ uint32_t half_of(const uint4& r, int n) {
  const uint32_t w = (n >> 1) == 0 ? r.x : (n >> 1) == 1 ? r.y : (n >> 1) == 2 ? r.z : r.w;
  return (n & 1) ? (w >> 16) : (w & 0xffffu);
}

// Registers (or global, scalar mode) -> LDS tile [ROWS][LDK], k contiguous.
template <int ROWS, int BK, int LDK>
__device__ __forceinline__ void commit(const View<bf16_t>& v, int k0, const Regs<ROWS, BK>& R,
                                       bf16_t* lds) {
  typedef Regs<ROWS, BK> RG;
  const int tid = threadIdx.x;
  if (!v.vec) {
    for (int e = tid; e < ROWS * BK; e += 256) {
      const int row = e / BK, kk = e % BK;
      lds[row * LDK + kk] = load_elem(v, row, k0 + kk);
    }
    return;
  }
  if (v.kcontig) {
#pragma unroll
    for (int i = 0; i < RG::PER_K; ++i) {
      const int c = tid + 256 * i;
      if (c < RG::CH) {
        const int row = c / RG::CPR, kc = c % RG::CPR;
        *reinterpret_cast<uint4*>(lds + row * LDK + kc * 8) = R.r[i];
      }
    }
  } else {
    constexpr int MNC = ROWS / 8;
#pragma unroll
    for (int i = 0; i < RG::PER_B; ++i) {
      const int b = tid + 256 * i;
      if (b < RG::NBLK) {
        const int mnc = b % MNC, kq = b / MNC;
#pragma unroll
        for (int n = 0; n < 8; ++n) {
          uint2 w;
          w.x = half_of(R.r[4 * i + 0], n) | (half_of(R.r[4 * i + 1], n) << 16);
          w.y = half_of(R.r[4 * i + 2], n) | (half_of(R.r[4 * i + 3], n) << 16);
          *reinterpret_cast<uint2*>(lds + (mnc * 8 + n) * LDK + kq * 4) = w;
        }
      }
    }
  }
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
template <int BM, int BN, int WM, int WN, int MODE, int EPI, bool PAIRED>
__global__ __launch_bounds__(256) void gemm_bf16(GemmArgs p) {
  constexpr int BK = 64, LDK = BK + 8;
  constexpr int WAVES_N = BN / WN, MF = WM / 32, NF = WN / 32;
  static_assert((BM / WM) * (BN / WN) == 4, "four waves per block");
  static_assert(!PAIRED || (NF % 2 == 0), "paired tiles need gate and up fragments");
  __shared__ __attribute__((aligned(16))) bf16_t smem[2 * (BM + BN) * LDK];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave / WAVES_N, wn = wave % WAVES_N;

  int e, n_tile, rows, m0 = 0, krows = 0;
  int64_t row0;
  if (MODE == GROUP_M) {
    const int mtot = *p.ntiles;
    const int total = mtot * p.ntn;
    if (static_cast<int>(blockIdx.x) >= total) return;
    const int L = xcd_remap(blockIdx.x, total);
    const int mt = L % mtot;
    n_tile = L / mtot;
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

  auto make_views = [&](int seg, View<bf16_t>& va, View<bf16_t>& vb) {
    const Opnd& A = p.a[seg];
    const Opnd& B = p.b[seg];
    va.ld = A.ld; va.kcontig = A.kcontig; va.vec = A.vec; va.paired = 0;
    vb.ld = B.ld; vb.kcontig = B.kcontig; vb.vec = B.vec; vb.paired = 0;
    if (MODE == GROUP_M) {
      va.base = static_cast<const bf16_t*>(A.ptr) + row0 * A.ld;
      va.klim = p.K[seg];
      va.mn_lim = rows;
      const bf16_t* wb = static_cast<const bf16_t*>(B.ptr) + static_cast<int64_t>(e) * B.estride;
      vb.klim = p.K[seg];
      if (PAIRED) {
        vb.base = wb;
        vb.paired = 1;
        vb.half = BN / 2;
        vb.pbase = n_tile * (BN / 2);
        vb.I = p.I;
        vb.mn_lim = BN;
      } else {
        vb.base = B.kcontig ? wb + static_cast<int64_t>(n0) * B.ld : wb + n0;
        vb.mn_lim = p.N - n0;
      }
    } else {
      va.base = static_cast<const bf16_t*>(A.ptr) + row0 * A.ld + m0;
      va.klim = krows;
      va.mn_lim = p.M - m0;
      vb.base = static_cast<const bf16_t*>(B.ptr) + row0 * B.ld + n0;
      vb.klim = krows;
      vb.mn_lim = p.N - n0;
    }
  };

  const int nk0 = MODE == GROUP_M ? (p.K[0] + BK - 1) / BK : (krows + BK - 1) / BK;
  const int nk1 = MODE == GROUP_M ? (p.K[1] + BK - 1) / BK : 0;
  const int nk = nk0 + nk1;

  f32x16 acc[MF][NF];
#pragma unroll
  for (int i = 0; i < MF; ++i)
#pragma unroll
    for (int j = 0; j < NF; ++j)
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[i][j][v] = 0.f;

  Regs<BM, BK> ra;
  Regs<BN, BK> rb;
  View<bf16_t> va, vb;
  int seg = 0, k0 = 0;
  if (nk > 0) {
    seg = nk0 > 0 ? 0 : 1;
    k0 = 0;
    make_views(seg, va, vb);
    fetch<BM, BK>(va, k0, ra);
    fetch<BN, BK>(vb, k0, rb);
    commit<BM, BK, LDK>(va, k0, ra, smem);
    commit<BN, BK, LDK>(vb, k0, rb, smem + BM * LDK);
  }
  __syncthreads();

  for (int it = 0; it < nk; ++it) {
    const int cur = it & 1;
    const int kvalid = (seg == 0 ? (MODE == GROUP_M ? p.K[0] : krows) : p.K[1]) - k0;
    View<bf16_t> na, nb;
    int nseg = seg, nk0v = k0;
    const bool has_next = it + 1 < nk;
    if (has_next) {
      if (it + 1 < nk0) {
        nseg = 0;
        nk0v = (it + 1) * BK;
      } else {
        nseg = 1;
        nk0v = (it + 1 - nk0) * BK;
      }
      make_views(nseg, na, nb);
      fetch<BM, BK>(na, nk0v, ra);
      fetch<BN, BK>(nb, nk0v, rb);
    }

    const bf16_t* sA = smem + cur * (BM + BN) * LDK;
    const bf16_t* sB = sA + BM * LDK;
#pragma unroll
    for (int ks = 0; ks < BK / 16; ++ks) {
      if (ks * 16 < kvalid) {
        bf16x8 af[MF], bf[NF];
        const int kof = ks * 16 + (lane >> 5) * 8;
#pragma unroll
        for (int mi = 0; mi < MF; ++mi)
          af[mi] = *reinterpret_cast<const bf16x8*>(sA + (wm * WM + mi * 32 + (lane & 31)) * LDK + kof);
#pragma unroll
        for (int ni = 0; ni < NF; ++ni) {
          int nr;
          if (PAIRED)
            nr = (ni < NF / 2) ? wn * (WN / 2) + ni * 32 : BN / 2 + wn * (WN / 2) + (ni - NF / 2) * 32;
          else
            nr = wn * WN + ni * 32;
          bf[ni] = *reinterpret_cast<const bf16x8*>(sB + (nr + (lane & 31)) * LDK + kof);
        }
#pragma unroll
        for (int mi = 0; mi < MF; ++mi)
#pragma unroll
          for (int ni = 0; ni < NF; ++ni)
            acc[mi][ni] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(bf[ni], af[mi], acc[mi][ni], 0, 0, 0);
      }
    }

    if (has_next) {
      bf16_t* dA = smem + (cur ^ 1) * (BM + BN) * LDK;
      commit<BM, BK, LDK>(na, nk0v, ra, dA);
      commit<BN, BK, LDK>(nb, nk0v, rb, dA + BM * LDK);
      seg = nseg;
      k0 = nk0v;
    }
    __syncthreads();
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
    if (d.r <= 32)
      return launch(gemm_bf16<128, 32, 32, 32, GROUP_M, EPI_STORE, false>, gm_grid(d, 1), a, s);
    return launch(gemm_bf16<128, 64, 32, 64, GROUP_M, EPI_STORE, false>, gm_grid(d, 1), a, s);
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
        return launch(gemm_bf16<256, 32, 64, 32, GROUP_K, EPI_STORE, false>, d.E * a.ntm, a, s);
      }
      a.ntm = ceil_div(P, 256);
      return launch(gemm_bf16<256, 64, 64, 64, GROUP_K, EPI_STORE, false>, d.E * a.ntm, a, s);
    }
    // [r, big] (or both small)
    a.ntn = ceil_div(Q, 256);
    if (P <= 32) {
      a.ntm = 1;
      return launch(gemm_bf16<32, 256, 32, 64, GROUP_K, EPI_STORE, false>, d.E * a.ntn, a, s);
    }
    a.ntm = ceil_div(P, 64);
    return launch(gemm_bf16<64, 256, 64, 64, GROUP_K, EPI_STORE, false>, d.E * a.ntm * a.ntn, a,
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
      MOE_TRY(launch(gemm_bf16<128, 256, 64, 128, GROUP_M, EPI_SWIGLU, true>, gm_grid(d, a.ntn),
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
      MOE_TRY(launch(gemm_bf16<128, 256, 64, 128, GROUP_M, EPI_STORE, false>, gm_grid(d, a.ntn),
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
      MOE_TRY(launch(gemm_bf16<128, 256, 64, 128, GROUP_M, EPI_SWIGLU_BWD, false>,
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
      MOE_TRY(launch(gemm_bf16<128, 256, 64, 128, GROUP_M, EPI_STORE, false>, gm_grid(d, a.ntn),
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
