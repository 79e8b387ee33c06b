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
//  - GROUP_KV: GROUP_K for dB = D^T U that also forms, from the D rows it
//    already holds in LDS, float32 partials of the side product D B over its
//    feature tile (summed over tiles by a second kernel), so that D is read
//    once for both.
// Operands are staged through LDS in 16-byte chunks, in the layout they have
// in memory (k-contiguous or output-contiguous, XOR-swizzled); fragments of
// output-contiguous tiles are read with the gfx950 transpose read. 16-bit
// products use v_mfma_f32_32x32x16_bf16 (or _f16) with float32 accumulation;
// the weight fragment is the MFMA A operand so that each lane ends up holding
// consecutive output columns of one row. float32 layers use a plain FMA
// kernel with the same tiling logic.
#include <stdlib.h>

#include <algorithm>
#include <type_traits>

#include "device_common.h"
#include "launch.h"

namespace moe {

namespace {

enum Mode { GROUP_M = 0, GROUP_K = 1, GROUP_KV = 2 };
// EPI_STORE_F32: float32 output (router logits); EPI_ADD: out = src + result
// with src = aux when given (merged export: W + s B A) else out itself (an
// accumulate); the sum formed in float32, one rounding.
enum Epi { EPI_STORE = 0, EPI_SWIGLU = 1, EPI_SWIGLU_BWD = 2, EPI_STORE_F32 = 3, EPI_ADD = 4 };

struct Opnd {
  const void* ptr;
  int64_t estride;  // elements between consecutive experts (0: not per expert)
  int64_t ld;       // leading dimension in elements
  int kcontig;      // 1: (mn, k) at ptr[mn*ld + k]; 0: at ptr[k*ld + mn]
  int vec;          // 16-byte chunks allowed (alignment and extents are multiples of 8)
  // Gathered rows (the layer input read in token order): row i of the
  // permuted order is row rows[i] / rows_div of ptr, which holds rows_bytes
  // bytes. Null rows: the operand's rows are in permuted order. Gathered
  // are the A operand of GROUP_M (rows along mn: x or dY) and, in the weight
  // gradients, the operand whose rows run along k (dY as A of dB_d, x as B of
  // dA_gu and dW_gu).
  const int32_t* rows;
  int rows_div;
  int64_t rows_bytes;
};

struct GemmArgs {
  Opnd a[2], b[2];  // [0] main segment, [1] LoRA segment (GROUP_M only)
  int K[2];         // GROUP_M: K extent of each segment (K[1] may be 0)
  int M, N;         // GROUP_K: output extent; GROUP_M: N = output columns (features)
  int E;
  const int32_t* offsets;  // [E+1]
  const int4* tiles;       // GROUP_M: {expert, first row, valid rows, raster group}
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
  int dtype;  // host side only: MOE_BF16 or MOE_F16 picks the 16-bit kernel
  // GROUP_KV: B of the side product (per expert [M, N] row-major, expert e of
  // the launch uses B[e / vsplit]) and its float32 partials vp[M tile][row][N]
  const void* vb;
  int64_t vb_estride;
  float* vp;
  int64_t vp_tstride;  // elements between M tiles of vp
  int vsplit;
  // EPI_SWIGLU_BWD (GROUP_M), both optional: roww[row] scales the product
  // before the SwiGLU derivative (dAct = w * acc); dwp receives, per output
  // row, float32 partial sums of acc * act over each wave's column slice
  // (at dwp[row * dwp_slots + n_tile * (BN / WN) + wave column]), act being
  // SwiGLU(h) recomputed from the h the epilogue loads.
  const float* roww;
  float* dwp;
  int dwp_slots;
};

// Spread `total` logical tiles over the 8 XCDs so that each XCD works on a
// contiguous range of them (workgroup b is dispatched to XCD b % 8).
__device__ __forceinline__ int xcd_remap(int b, int total) {
  const int x = b & 7, j = b >> 3, q = total >> 3, rem = total & 7;
  return x * q + (x < rem ? x : rem) + j;
}

// Tile-list entries are {expert, first row, valid rows, group}: an expert's M
// tiles form groups of at most 8 consecutive entries, and `group` holds the
// group's first entry times 16 plus its size. Logical tiles L = gs * ntn ..
// (gs + gsz) * ntn - 1 belong to the group starting at entry gs, M tile
// fastest, so L / ntn is always one of that group's entries. Returns the
// entry of logical tile L and sets its N tile.
constexpr int kTileGroup = 8;
__device__ __forceinline__ int group_tile(const int4* tiles, int L, int ntn, int& n_tile) {
  const int g = tiles[L / ntn].w;
  const int gs = g >> 4, gsz = g & 15;
  const int rem = L - gs * ntn;
  n_tile = rem / gsz;
  return gs + rem % gsz;
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
  // gathered rows (Opnd::rows from this tile's first row on, and its divisor):
  // mn (k-contiguous) or k (output-contiguous) index i is row grow[i] / gk of base
  const int32_t* grow;
  int gk;
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
__device__ __forceinline__ int64_t gathered_row(const View<T>& v, int64_t i) {
  return v.grow ? static_cast<int64_t>(static_cast<uint32_t>(v.grow[i]) / static_cast<uint32_t>(v.gk))
                : i;
}

template <typename T>
__device__ __forceinline__ T load_elem(const View<T>& v, int n, int k) {
  bool ok;
  const int64_t g = map_mn(v, n, ok);
  if (!ok || k >= v.klim) return T(0);
  return v.kcontig ? v.base[gathered_row(v, g) * v.ld + k]
                   : v.base[gathered_row(v, k) * v.ld + g];
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
    if (EPI == EPI_STORE || EPI == EPI_STORE_F32 || EPI == EPI_ADD) {
      float o[4];
      T* rp = static_cast<T*>(p.out) + row * p.ld_out;
      const T* sp = EPI == EPI_ADD && p.aux ? static_cast<const T*>(p.aux) + row * p.ld_aux : rp;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        o[j] = v[j] * p.scale;
        if (EPI == EPI_ADD && n_col + j < p.N) o[j] += to_f32<T>(sp[n_col + j]);
      }
      store4<T>(rp, n_col, p.N, (p.ld_out & 3) == 0, o);
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
// LDS tiles are BK (32 or 64) deep in k, unpadded, with 16-byte-chunk XOR swizzles:
//   k-contiguous tile [R][BK]: row r keeps k-chunk c at position c ^ kswz<BK>(r)
//   n-contiguous tile [BK][R]: k-row k keeps n-chunk c at position c ^ nswz<R>(k)
// chosen so that every 256-byte group of a fragment read (16 lanes of
// ds_read_b128, 32 lanes of ds_read_b64_tr_b16) touches each LDS bank once.
// Both layouts yield the same MFMA fragment: lane l holds 8 consecutive k
// (block l/32) of the row or column l%32 (the transpose read, CDNA4's
// ds_read_b64_tr_b16, gathers them from the k-major tile). Tiles are filled by
// buffer->LDS DMA with no register staging: each wave instruction writes 1 KB
// of LDS, lane l at +16 l, from a per-lane byte offset that encodes the
// swizzle; lanes outside the operand get an out-of-range offset and the
// hardware writes zeros. NST LDS stages keep NST-1 tiles in flight while one
// is multiplied.
constexpr uint32_t kOOB = 0x80000000u;

typedef __attribute__((address_space(3))) void lds_void;
typedef short v4s __attribute__((ext_vector_type(4)));
typedef short v8s __attribute__((ext_vector_type(8)));

template <int BK>
__device__ __forceinline__ int kswz(int row) {
  return BK == 64 ? ((row >> 1) & 7) : ((row >> 2) & 3);
}

template <int R>
__device__ __forceinline__ int nswz(int k) {
  return R >= 128 ? ((k & 3) << 2) : (R == 64 ? (((k >> 1) & 1) << 2) : 0);
}

template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}

// Own LDS traffic finished, then a workgroup barrier.
__device__ __forceinline__ void barrier_lds() {
  asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

// Buffer resource (V#) over [base, base + nrec bytes): raw, stride 0.
__device__ __forceinline__ u32x4 buffer_rsrc(const void* base, int nrec) {
  const uint64_t b = reinterpret_cast<uint64_t>(base);
  u32x4 r;
  r[0] = static_cast<uint32_t>(b);
  r[1] = static_cast<uint32_t>(b >> 32) & 0xffffu;
  r[2] = static_cast<uint32_t>(nrec);
  r[3] = 0x00020000u;
  return r;
}

// 16 bytes per lane, global -> LDS: lane l's bytes land at lds + 16 l. The
// instruction is issued from inline asm so that the compiler does not treat
// it as an LDS store it must wait for before every later LDS read (it would
// insert s_waitcnt vmcnt(0) and drain all tiles in flight); completion is
// tracked by the explicit vmcnt waits of the pipeline instead. The asm has no
// outputs, so no register is ever written by a load still in flight.
__device__ __forceinline__ void dma16(const char* lds, const u32x4& rs, uint32_t vo,
                                      uint32_t soff) {
  const uint32_t m0 = __builtin_amdgcn_readfirstlane(static_cast<uint32_t>(
      reinterpret_cast<uintptr_t>((__attribute__((address_space(3))) const char*)(lds))));
  // resource and offset are wave-uniform; make that explicit for the SGPR operands
  u32x4 srs;
  srs[0] = __builtin_amdgcn_readfirstlane(rs[0]);
  srs[1] = __builtin_amdgcn_readfirstlane(rs[1]);
  srs[2] = __builtin_amdgcn_readfirstlane(rs[2]);
  srs[3] = __builtin_amdgcn_readfirstlane(rs[3]);
  const uint32_t ssoff = __builtin_amdgcn_readfirstlane(soff);
  // s_nop 4: the resource/offset SGPRs may have just been written by VALU
  // (v_readfirstlane), which a VMEM read may only follow after 5 wait states,
  // and M0 needs 1 wait state before an LDS DMA; the compiler's hazard
  // recognizer does not look inside inline asm, so the asm provides both.
  asm volatile("s_nop 4\n\tbuffer_load_dwordx4 %1, %2, %3 offen lds" ::"{m0}"(m0), "v"(vo),
               "s"(srs), "s"(ssoff)
               : "memory");
}

__device__ __forceinline__ int clamp_records(int64_t bytes) {
  return bytes <= 0 ? 0 : (bytes > 0x7fffffff ? 0x7fffffff : static_cast<int>(bytes));
}

// Fill geometry of one operand tile of ROWS rows (or columns) x BK, filled
// by NW waves in 1 KB wave instructions (16 bytes per lane).
template <int ROWS, int BK, bool KC, int NW>
struct Geo {
  static constexpr int TI = ROWS * BK * 2 / 1024;  // 1 KB instructions per tile
  static constexpr int NIW = (TI + NW - 1) / NW;   // per wave (upper bound)
  static constexpr int MINW = TI / NW;             // issued by every wave
  static constexpr int CPR = KC ? BK / 8 : ROWS / 8;        // chunks per LDS row
  static constexpr int RPI = KC ? 512 / BK : 512 / ROWS;    // LDS rows per instruction
};

// DMA plan of one operand tile: buffer (base, bytes), per-instruction lane offsets.
template <int ROWS, int BK, bool KC, int NW>
struct Plan {
  const void* base;
  int64_t bytes;  // extent of the operand from base
  int nrec;
  u32x4 rs;  // buffer resource over [base, base + nrec)
  uint32_t vo[Geo<ROWS, BK, KC, NW>::NIW];
  int vec;
  int klim;
  int64_t ld;
  View<bf16_t> view;  // element view for the slow (non-DMA) fill
};

template <int ROWS, int BK, bool KC, int NW>
__device__ __forceinline__ void make_plan(Plan<ROWS, BK, KC, NW>& P, const View<bf16_t>& v,
                                          int64_t bytes, int vec, int wave, int lane) {
  typedef Geo<ROWS, BK, KC, NW> G;
  P.view = v;
  P.vec = vec;
  P.klim = v.klim;
  P.ld = v.ld;
  P.base = v.base;
  P.bytes = bytes;
  P.nrec = clamp_records(bytes);
  P.rs = buffer_rsrc(v.base, P.nrec);
#pragma unroll
  for (int i = 0; i < G::NIW; ++i) {
    const int j = wave + NW * i;  // instruction index within the tile
    const int r = G::RPI * j + lane / G::CPR;
    const int p = lane % G::CPR;
    uint32_t vo = kOOB;
    if (KC) {
      const int c = p ^ kswz<BK>(r);
      bool ok;
      const int64_t g = map_mn(v, r, ok);
      if (ok && r < ROWS) vo = static_cast<uint32_t>((gathered_row(v, g) * v.ld + c * 8) * 2);
    } else {
      // gathered: the offsets depend on the k tile's rows (gather_vo)
      const int cn = p ^ nswz<ROWS>(r);
      if (cn * 8 < v.mn_lim && r < BK && !v.grow) vo = static_cast<uint32_t>((r * v.ld + cn * 8) * 2);
    }
    P.vo[i] = vo;
  }
}

// Buffer resource and scalar offset of the tile at k0. A k-contiguous
// operand keeps one resource (k0 is a small byte offset). An output-contiguous
// one advances along its rows: its resource starts at row k0 (64-bit address
// arithmetic) and covers the rest of the operand, so neither the 32-bit scalar
// offset nor the 2^31-byte record count limits how many rows it spans (a
// weight gradient runs over all of an expert's rows).
template <int ROWS, int BK, bool KC, int NW>
__device__ __forceinline__ u32x4 tile_rsrc(const Plan<ROWS, BK, KC, NW>& P, int k0,
                                           uint32_t& soff) {
  if (KC) {
    soff = static_cast<uint32_t>(k0) * 2;
    return P.rs;
  }
  soff = 0;
  if (P.view.grow) return P.rs;  // gathered rows: per-lane offsets from the start
  const int64_t adv = static_cast<int64_t>(k0) * P.ld * 2;
  return buffer_rsrc(static_cast<const char*>(P.base) + adv, clamp_records(P.bytes - adv));
}

// Lane offset of instruction j of an output-contiguous tile at k0 whose rows
// are gathered: the instruction covers the tile's k rows RPI*j .. RPI*j+RPI-1
// (wave-uniform), whose row numbers come in through scalar loads (constant
// address space: they go through the scalar cache and are counted apart from
// the DMA loads in flight), so the DMA pipeline's vector-memory waits stay
// exact. table (optional): the byte offsets of the block's rows from row tw0
// on, in LDS (read instead of the scalar loads).
template <int ROWS, int BK, bool KC, int NW>
__device__ __forceinline__ uint32_t gather_vo(const Plan<ROWS, BK, KC, NW>& P, int k0, int j,
                                              int lane, const uint32_t* table = nullptr,
                                              int tw0 = 0) {
  typedef Geo<ROWS, BK, KC, NW> G;
  typedef const __attribute__((address_space(4))) int32_t* cptr;
  if (P.klim <= 0) return kOOB;
  const int r0 = k0 + G::RPI * j, last = P.klim - 1, t = lane / G::CPR;
  const int cn = (lane % G::CPR) ^ nswz<ROWS>(G::RPI * j + t);
  if (table) {
    const uint32_t off = table[min(r0 + t, last) - tw0];
    if (r0 + t > last || cn * 8 >= P.view.mn_lim) return kOOB;
    return off + static_cast<uint32_t>(cn) * 16;
  }
  const cptr rows = (cptr)(P.view.grow);
  int sp = 0;
#pragma unroll
  for (int q = 0; q < G::RPI; ++q) {
    const int v = rows[min(r0 + q, last)];
    if (t == q) sp = v;
  }
  if (r0 + t > last || cn * 8 >= P.view.mn_lim) return kOOB;
  const uint32_t row = static_cast<uint32_t>(sp) / static_cast<uint32_t>(P.view.gk);
  return static_cast<uint32_t>((static_cast<int64_t>(row) * P.ld + cn * 8) * 2);
}

// Issue one tile: DMA when possible, else an element-wise fill. GATH false:
// the operand is never gathered along k (no code for it).
template <int ROWS, int BK, bool KC, int NW, bool GATH = true>
__device__ __forceinline__ void fill(const Plan<ROWS, BK, KC, NW>& P, int k0, char* lds, int wave,
                                     int lane, const uint32_t* gtab = nullptr, int tw0 = 0) {
  typedef Geo<ROWS, BK, KC, NW> G;
  if (P.vec) {
    uint32_t soff;
    const u32x4 rs = tile_rsrc(P, k0, soff);
    const bool tail = KC && (k0 + BK > P.klim);  // n-contiguous tails hit the buffer bound
#pragma unroll
    for (int i = 0; i < G::NIW; ++i) {
      const int j = wave + NW * i;
      if (G::TI % NW == 0 || j < G::TI) {
        uint32_t vo = P.vo[i];
        if (GATH && !KC && P.view.grow) vo = gather_vo(P, k0, j, lane, gtab, tw0);
        if (tail) {
          const int r = G::RPI * j + lane / G::CPR;
          const int c = (lane % G::CPR) ^ kswz<BK>(r);
          if (k0 + c * 8 >= P.klim) vo = kOOB;
        }
        dma16(lds + j * 1024, rs, vo, soff);
      }
    }
  } else {
    bf16_t* t = reinterpret_cast<bf16_t*>(lds);
    for (int e = threadIdx.x; e < ROWS * BK; e += 64 * NW) {
      int byte;
      bf16_t val;
      if (KC) {
        const int row = e / BK, k = e % BK;
        byte = row * BK * 2 + (((k >> 3) ^ kswz<BK>(row)) << 4) + (k & 7) * 2;
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

// One DMA instruction (index i of this wave's share) of a tile; DMA plans only.
// GIVEN: gvo is the lane offset, formed by the caller (the plan's own offset,
// or a gathered row's); GATH false: the operand is never gathered along k.
template <int ROWS, int BK, bool KC, int NW, bool GATH = true, bool GIVEN = false>
__device__ __forceinline__ void fill_one(const Plan<ROWS, BK, KC, NW>& P, int k0, char* lds,
                                         int wave, int lane, int i, uint32_t gvo = 0) {
  typedef Geo<ROWS, BK, KC, NW> G;
  const int j = wave + NW * i;
  if (G::TI % NW != 0 && j >= G::TI) return;
  uint32_t soff;
  const u32x4 rs = tile_rsrc(P, k0, soff);
  uint32_t vo = P.vo[i];
  if (GIVEN)
    vo = gvo;
  else if (GATH && !KC && P.view.grow)
    vo = gather_vo(P, k0, j, lane);
  if (KC && k0 + BK > P.klim) {  // k tail of a k-contiguous operand: mask by lane
    const int r = G::RPI * j + lane / G::CPR;
    const int c = (lane % G::CPR) ^ kswz<BK>(r);
    if (k0 + c * 8 >= P.klim) vo = kOOB;
  }
  dma16(lds + j * 1024, rs, vo, soff);
}

// A fill geometry tagged with its operand's k-contiguity (for generic lambdas).
template <typename G, bool KC>
struct GeoK : G {
  static constexpr bool KCV = KC;
};

// Per-lane LDS byte offsets of the MFMA fragments.
template <int ROWS, int BK, bool KC, int NFR>
struct FragAddr {
  int off[KC ? BK / 16 : NFR];  // KC: per k-step (shared by all fragments); NC: per fragment
};

template <int ROWS, int BK, bool KC, int NFR>
__device__ __forceinline__ void frag_addr(FragAddr<ROWS, BK, KC, NFR>& F,
                                          const int (&fr_base)[NFR], int lane) {
  if (KC) {
    const int h = lane >> 5, r = lane & 31;
#pragma unroll
    for (int ks = 0; ks < BK / 16; ++ks)
      F.off[ks] = r * BK * 2 + ((((2 * ks + h) ^ kswz<BK>(r))) << 4);
  } else {
    const int G = lane >> 4, li = lane & 15;
    const int kl = (G >> 1) * 8 + (li >> 2);  // k row of this lane in a k-step (first read)
#pragma unroll
    for (int f = 0; f < (KC ? 0 : NFR); ++f) {
      const int n = fr_base[f] + (G & 1) * 16 + (li & 3) * 4;
      F.off[KC ? 0 : f] = kl * ROWS * 2 + ((((n >> 3) ^ nswz<ROWS>(kl))) << 4) + (n & 7) * 2;
    }
  }
}

template <int ROWS, int BK, bool KC, int NFR>
__device__ __forceinline__ bf16x8 read_frag(const char* tile,
                                            const FragAddr<ROWS, BK, KC, NFR>& F, int f,
                                            int fr_base_f, int ks) {
  if (KC) {
    return *reinterpret_cast<const bf16x8*>(tile + fr_base_f * BK * 2 + F.off[ks]);
  } else {
    const char* p = tile + F.off[KC ? 0 : f] + ks * 16 * ROWS * 2;
    v4s lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) v4s*)(p));
    v4s hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
        (__attribute__((address_space(3))) v4s*)(p + 4 * ROWS * 2));
    v8s r = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
    return __builtin_bit_cast(bf16x8, r);
  }
}

// ---- epilogue staging helpers
// A wave's float32 slab is 32 rows x WN columns; row r keeps 16-byte chunk c
// at c ^ sswz(r), so that 16 lanes writing one chunk column of 16 rows, or
// reading 16 row segments, hit distinct LDS banks.
template <int WN>
__device__ __forceinline__ int slab_off(int r, int c) {
  const int sw = WN >= 64 ? (r & 15) : ((r >> 1) & 7);
  return r * WN * 4 + ((c ^ sw) << 4);
}

// Eight floats: chunks c and c+1 of row r.
template <int WN>
__device__ __forceinline__ void read8(const char* slab, int r, int c, float (&v)[8]) {
  const f32x4 lo = *reinterpret_cast<const f32x4*>(slab + slab_off<WN>(r, c));
  const f32x4 hi = *reinterpret_cast<const f32x4*>(slab + slab_off<WN>(r, c + 1));
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    v[j] = lo[j];
    v[4 + j] = hi[j];
  }
}

// Columns 8s..8s+7 of row r. Lanes of the upper half of a row read their odd
// chunk first, so that 16 lanes of either read touch 16 distinct 16-byte bank groups.
template <int WN>
__device__ __forceinline__ void read8_interleaved(const char* slab, int r, int s, float (&v)[8]) {
  const int odd = s >= WN / 16 ? 1 : 0;
  const f32x4 x = *reinterpret_cast<const f32x4*>(slab + slab_off<WN>(r, 2 * s + odd));
  const f32x4 y = *reinterpret_cast<const f32x4*>(slab + slab_off<WN>(r, 2 * s + (odd ^ 1)));
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    v[j] = odd ? y[j] : x[j];
    v[4 + j] = odd ? x[j] : y[j];
  }
}

// ---- the two 16-bit storage formats: bfloat16 and IEEE half, both held as
// raw 16-bit words (the tiles, DMA and LDS layouts do not care which); F16
// selects the MFMA instruction and the conversions of the epilogue.
template <bool F16>
__device__ __forceinline__ float h16_to_f32(uint16_t v) {
  if constexpr (F16) return static_cast<float>(__builtin_bit_cast(_Float16, v));
  else return __uint_as_float(static_cast<uint32_t>(v) << 16);
}

template <bool F16>
__device__ __forceinline__ uint16_t f32_to_h16(float f) {  // round to nearest even
  if constexpr (F16) return __builtin_bit_cast(uint16_t, static_cast<_Float16>(f));
  else return f32_to_bf16(f);
}

typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));

// acc += A B^T on a 32 x 32 tile, k = 16 (bfloat16 or half operands, float32 accumulate)
template <bool F16>
__device__ __forceinline__ f32x16 mfma32(bf16x8 a, bf16x8 b, f32x16 c) {
  if constexpr (F16)
    return __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(f16x8, a),
                                                  __builtin_bit_cast(f16x8, b), c, 0, 0, 0);
  else
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

// Eight consecutive 16-bit values as one 16-byte global access (16-byte aligned).
// Epilogue traffic is streamed once: non-temporal loads and stores keep it
// from evicting the operand tiles the other blocks are reading from L2.
template <bool F16>
__device__ __forceinline__ void unpack8(const u32x4& r, float (&v)[8]) {
  const uint32_t w[4] = {r[0], r[1], r[2], r[3]};
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    v[2 * j] = h16_to_f32<F16>(static_cast<uint16_t>(w[j] & 0xffffu));
    v[2 * j + 1] = h16_to_f32<F16>(static_cast<uint16_t>(w[j] >> 16));
  }
}

template <bool F16>
__device__ __forceinline__ void load8(const bf16_t* p, float (&v)[8]) {
  unpack8<F16>(__builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p)), v);
}

template <bool F16>
__device__ __forceinline__ void store8(bf16_t* p, const float (&v)[8]) {
  uint32_t w[4];
#pragma unroll
  for (int j = 0; j < 4; ++j)
    w[j] = static_cast<uint32_t>(f32_to_h16<F16>(v[2 * j])) |
           (static_cast<uint32_t>(f32_to_h16<F16>(v[2 * j + 1])) << 16);
  u32x4 q;
  q[0] = w[0];
  q[1] = w[1];
  q[2] = w[2];
  q[3] = w[3];
  __builtin_nontemporal_store(q, reinterpret_cast<u32x4*>(p));
}

// LDS writes of this wave are complete (and not reordered by the compiler)
// before its lanes read what other lanes wrote.
__device__ __forceinline__ void wave_lds_sync() { asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory"); }

template <bool F16, int BM, int BN, int WM, int WN, int BK, int NST, int MINB, int MODE, int EPI,
          bool PAIRED, bool A_KC, bool B_KC, int VST, int GATH = 0>
__global__ __launch_bounds__((BM / WM) * (BN / WN) * 64, MINB) void gemm16(GemmArgs p) {
  constexpr int WAVES_N = BN / WN, MF = WM / 32, NF = WN / 32;
  constexpr int NW = (BM / WM) * (BN / WN);
  constexpr int A_BYTES = BM * BK * 2, B_BYTES = BN * BK * 2, ST = A_BYTES + B_BYTES;
  typedef Geo<BM, BK, A_KC, NW> GA;
  typedef Geo<BN, BK, B_KC, NW> GB;
  static_assert(NW == 4 || NW == 8, "four or eight waves per block");
  static_assert(!PAIRED || (NF % 2 == 0), "paired tiles need gate and up fragments");
  static_assert(GA::TI >= 1 && GB::TI >= 1, "tile smaller than one DMA instruction");
  static_assert(VST || (NST >= 3 && NST <= 6 && (NST - 2) * (GA::MINW + GB::MINW) <= 63),
                "vmcnt range");
  // GROUP_KV: + the block's [BM][32] tile of the side-product B
  constexpr int VB_BYTES = MODE == GROUP_KV ? BM * 32 * 2 : 0;
  // GATH (weight gradients, DMA tiles): the reduction rows of operand A
  // (GATH 1: dY's rows for the B gradient of down) or B (GATH 2: x's rows for
  // the LoRA A gradient of gate_up and dW_gu) are read through a row list, so
  // that operand's lane offsets depend on each k tile's rows: they are formed
  // a k tile ahead from a table in LDS of the byte offsets of up to GT_ROWS
  // of the block's rows (sized so that two blocks still fit a CU). A
  // separate instantiation keeps the ungathered loop as it is.
  constexpr bool GK = MODE == GROUP_K || MODE == GROUP_KV;
  static_assert(GATH == 0 || (GK && VST == 0 && !A_KC && !B_KC), "gathered rows: DMA weight gradients");
  constexpr bool GATHER_A = GATH == 1, GATHER_B = GATH == 2;
  constexpr int GT_ROWS = GATH == 0                ? 0
                          : (GATHER_B && BM <= 32) ? 4096
                          : (GATHER_A && BN <= 32) ? 2048
                                                   : 1024;
  __shared__ __attribute__((aligned(1024))) char smem[NST * ST + VB_BYTES + GT_ROWS * 4];

  const int tid = threadIdx.x, lane = tid & 63;
  // wave index as a wave-uniform (scalar) value, so that everything derived
  // from it (DMA destinations, resources) stays in SGPRs
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  // The second and later rows of waves are rotated along N: when only the
  // first column of waves holds valid columns (a narrow last N tile), its
  // waves sit on different SIMDs (wave w runs on SIMD w % 4).
  const int wm = wave / WAVES_N, wn = (wave % WAVES_N + wm) % WAVES_N;

  int e, n_tile, rows, m0 = 0, krows = 0;
  int64_t row0;
  if (MODE == GROUP_M) {
    const int mtot = *p.ntiles;
    const int total = mtot * p.ntn;
    if (static_cast<int>(blockIdx.x) >= total) return;
    // XCD-contiguous ranges, then groups of up to 8 M tiles of one expert
    // swept across all N tiles, so the tiles an XCD runs together share A
    // rows and the expert's weight columns in L2.
    const int L = xcd_remap(blockIdx.x, total);
    const int4 t = p.tiles[group_tile(p.tiles, L, p.ntn, n_tile)];
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

  // ---- DMA plans for the main segment (0) and the LoRA segment (1). Kept in
  // plain variables, never indexed by a runtime value, so they stay in
  // registers: a scratch access would bring an s_waitcnt vmcnt(0) that also
  // drains every tile in flight.
  Plan<BM, BK, A_KC, NW> pa0, pa1;
  Plan<BN, BK, B_KC, NW> pb0, pb1;
  auto build = [&](int seg, Plan<BM, BK, A_KC, NW>& PA, Plan<BN, BK, B_KC, NW>& PB) {
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
      if (A.rows) {
        va.base = static_cast<const bf16_t*>(A.ptr);
        va.grow = A.rows + row0;
        va.gk = A.rows_div;
        abytes = A.rows_bytes;
      }
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
      if (GATHER_A) {
        va.base = static_cast<const bf16_t*>(A.ptr) + m0;
        va.grow = A.rows + row0;
        va.gk = A.rows_div;
        abytes = A.rows_bytes - static_cast<int64_t>(m0) * 2;
      }
      vb.base = static_cast<const bf16_t*>(B.ptr) + row0 * B.ld + n0;
      vb.klim = krows;
      vb.mn_lim = p.N - n0;
      bbytes = static_cast<int64_t>(krows) * B.ld * 2 - static_cast<int64_t>(n0) * 2;
      if (GATHER_B) {
        vb.base = static_cast<const bf16_t*>(B.ptr) + n0;
        vb.grow = B.rows + row0;
        vb.gk = B.rows_div;
        bbytes = B.rows_bytes - static_cast<int64_t>(n0) * 2;
      }
    }
    make_plan<BM, BK, A_KC, NW>(PA, va, abytes, A.vec, wave, lane);
    make_plan<BN, BK, B_KC, NW>(PB, vb, bbytes, B.vec, wave, lane);
  };
  build(0, pa0, pb0);
  if (MODE == GROUP_M) {
    build(1, pa1, pb1);
  } else {
    pa1 = pa0;
    pb1 = pb0;
  }

  const int nk0 = MODE == GROUP_M ? (p.K[0] + BK - 1) / BK : (krows + BK - 1) / BK;
  const int nk1 = MODE == GROUP_M ? (p.K[1] + BK - 1) / BK : 0;
  const int nk = nk0 + nk1;
  const bool dma0 = pa0.vec && pb0.vec, dma1 = pa1.vec && pb1.vec;

  // Gathered reduction rows (GROUP_K, GROUP_KV): the byte offsets of the rows
  // from gw0 on in LDS, when formed, for the operand whose rows they are
  const uint32_t* gtab_a = nullptr;
  const uint32_t* gtab_b = nullptr;
  int gw0 = 0;
  auto issue = [&](int j) {  // a whole stage at once (prologue, element-wise fills)
    char* sa = smem + (j % NST) * ST;
    char* sb = sa + A_BYTES;
    if (j < nk0) {
      fill<BM, BK, A_KC, NW, GATHER_A>(pa0, j * BK, sa, wave, lane, gtab_a, gw0);
      fill<BN, BK, B_KC, NW, GATHER_B>(pb0, j * BK, sb, wave, lane, gtab_b, gw0);
    } else {
      fill<BM, BK, A_KC, NW, false>(pa1, (j - nk0) * BK, sa, wave, lane);
      fill<BN, BK, B_KC, NW, false>(pb1, (j - nk0) * BK, sb, wave, lane);
    }
  };
  // A stage filled only by DMA leaves at least MINW loads per operand outstanding.
  auto dma_stage = [&](int j) { return j < nk0 ? dma0 : dma1; };

  int fa_base[MF], fb_base[NF];
#pragma unroll
  for (int mi = 0; mi < MF; ++mi) fa_base[mi] = wm * WM + mi * 32;
#pragma unroll
  for (int ni = 0; ni < NF; ++ni) {
    if (PAIRED)
      fb_base[ni] = (ni < NF / 2) ? wn * (WN / 2) + ni * 32
                                  : BN / 2 + wn * (WN / 2) + (ni - NF / 2) * 32;
    else
      fb_base[ni] = wn * WN + ni * 32;
  }
  FragAddr<BM, BK, A_KC, MF> FA;
  FragAddr<BN, BK, B_KC, NF> FB;
  frag_addr<BM, BK, A_KC, MF>(FA, fa_base, lane);
  frag_addr<BN, BK, B_KC, NF>(FB, fb_base, lane);

  f32x16 acc[MF][NF];
#pragma unroll
  for (int i = 0; i < MF; ++i)
#pragma unroll
    for (int j = 0; j < NF; ++j)
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[i][j][v] = 0.f;

  // GROUP_KV: this block's feature rows of the expert's side-product B, as
  // MFMA fragments over the whole tile (k = feature, n = column of B; lane l
  // holds column l%32 and features 8(l/32)..+7 of each 16-feature step). The
  // [BM][32] tile goes through LDS in 16-byte pieces (zero-padded past M and
  // N; rows of B are 16-byte aligned, N a multiple of 8) and is read back
  // with transpose reads, like any output-contiguous operand.
  static_assert(MODE != GROUP_KV || (BM == 256 && BN == 32 && BK == 32 && !A_KC && VST == 0),
                "side-product partials assume 256 x 32 tiles, 32 rows per k tile");
  constexpr int VKS = MODE == GROUP_KV ? BM / 16 : 1;
  bf16x8 vbf[VKS];
  if constexpr (MODE == GROUP_KV) {
    const bf16_t* bm = static_cast<const bf16_t*>(p.vb) +
                       static_cast<int64_t>(e / p.vsplit) * p.vb_estride;
    char* vt = smem + NST * ST;
    for (int i = tid; i < BM * 4; i += NW * 64) {  // piece i: feature i/4, columns 8 (i%4)..
      const int f = i >> 2, c = i & 3;
      u32x4 v = {0u, 0u, 0u, 0u};
      if (m0 + f < p.M && c * 8 < p.N)
        v = *reinterpret_cast<const u32x4*>(bm + static_cast<int64_t>(m0 + f) * p.N + c * 8);
      *reinterpret_cast<u32x4*>(vt + f * 64 + c * 16) = v;
    }
    __syncthreads();
    FragAddr<32, BM, false, 1> FV;
    const int zero[1] = {0};
    frag_addr<32, BM, false, 1>(FV, zero, lane);
#pragma unroll
    for (int kk = 0; kk < VKS; ++kk) vbf[kk] = read_frag<32, BM, false, 1>(vt, FV, 0, 0, kk);
  }

  if constexpr (VST > 0) {
    // ---- Register-staged main loop: every wave loads its share of a k tile
    // into VGPRs (16 bytes per lane per 1 KB piece, the same lane offsets as
    // the DMA plans, out-of-range lanes read zeros) and writes it to the LDS
    // slot the tile belongs to. Two LDS slots and one register buffer: tile
    // it+1 is written during tile it's second k-step (its slot was last read
    // before the previous barrier), and the load of tile it+2 is issued into
    // the buffer just freed, so each load has a whole k tile of MFMAs to
    // arrive. Tile 1 is loaded together with tile 0 into a prologue-only
    // buffer (the accumulators hold nothing yet, so their registers are
    // free): a block waits for one load latency before its first MFMA.
    //
    // The steady state (the tiles whose staged load is a whole in-range tile
    // of the main segment) runs two tiles per iteration, so the LDS slot of
    // every access is a compile-time constant: fragment reads and staging
    // writes take their whole offset in the instruction's immediate field
    // from loop-invariant per-lane bases, and the loads need no masking.
    // The first tile, the tiles around the LoRA segment and the K tail, and
    // the last tile take the general path (slot chosen at run time, loads
    // masked).
    static_assert(VST == 1, "one register buffer");
    static_assert(NST == 2, "register staging uses two LDS slots");
    constexpr int KS = BK / 16;
    static_assert(KS % 2 == 0, "fragment double-buffering alternates per k-step");
    u32x4 ra[GA::NIW], rb[GB::NIW];
    // Buffer resource of a plan (wave-uniform: built in SGPRs).
    auto make_rs = [&](const auto& P) __attribute__((always_inline)) {
      // readfirstlane returns int: widen through uint32_t, never by sign extension
      const uint64_t base = reinterpret_cast<uint64_t>(P.base);
      const uint64_t lo = static_cast<uint32_t>(
          __builtin_amdgcn_readfirstlane(static_cast<uint32_t>(base)));
      const uint64_t hi = static_cast<uint32_t>(
          __builtin_amdgcn_readfirstlane(static_cast<uint32_t>(base >> 32)));
      return __builtin_amdgcn_make_buffer_rsrc(reinterpret_cast<void*>((hi << 32) | lo),
                                               static_cast<short>(0),
                                               __builtin_amdgcn_readfirstlane(P.nrec), 0x00020000);
    };
    __amdgpu_buffer_rsrc_t rsa = make_rs(pa0), rsb = make_rs(pb0);
    // CLEAN: the tile is a whole, in-range tile of the current plans (no
    // masking, every lane's offset as planned)
    auto vload = [&](auto& P, const __amdgpu_buffer_rsrc_t& rs, int k0, u32x4* r, auto geo,
                     bool live, auto cleanc) __attribute__((always_inline)) {
      typedef decltype(geo) G;
      constexpr bool CLEAN = decltype(cleanc)::value;
      const bool kc = decltype(geo)::KCV;
      const uint32_t soff = kc ? static_cast<uint32_t>(k0) * 2
                               : static_cast<uint32_t>(static_cast<int64_t>(k0) * P.ld * 2);
      const bool tail = !CLEAN && kc && (k0 + BK > P.klim);
#pragma unroll
      for (int i = 0; i < G::NIW; ++i) {
        const int j = wave + NW * i;
        if (G::TI % NW == 0 || j < G::TI) {
          uint32_t vo = P.vo[i];
          if constexpr (!CLEAN) {
            if (!live) vo = kOOB;
            if (tail) {
              const int rr = G::RPI * j + lane / G::CPR;
              const int c = (lane % G::CPR) ^ kswz<BK>(rr);
              if (k0 + c * 8 >= P.klim) vo = kOOB;
            }
          }
          r[i] = __builtin_amdgcn_raw_buffer_load_b128(rs, vo, __builtin_amdgcn_readfirstlane(soff), 0);
        }
      }
    };
    // Branch-free issue: the plans switch to the LoRA segment's once, before
    // its first tile is loaded (tiles are loaded in order), and live = false
    // issues the loads with every lane out of range (they return zeros and
    // touch no memory) instead of skipping them, so every path issues the
    // same loads and the compiler's waits stay exact.
    auto switch_plans = [&]() __attribute__((always_inline)) {
      pa0 = pa1;
      pb0 = pb1;
      rsa = make_rs(pa0);
      rsb = make_rs(pb0);
    };
    auto load_tile = [&](int j, u32x4* a, u32x4* b, bool live, auto cleanc) __attribute__((always_inline)) {
      const int k0 = (j >= nk0 ? j - nk0 : j) * BK;
      vload(pa0, rsa, k0, a, GeoK<GA, A_KC>(), live, cleanc);
      vload(pb0, rsb, k0, b, GeoK<GB, B_KC>(), live, cleanc);
    };
    // LDS layout [A slot 0 | A slot 1 | B slot 0 | B slot 1]: every access of
    // a slot lies within 64 KB of its operand's region start, so a per-lane
    // base register plus the instruction's immediate offset reaches it.
    constexpr int B_REGION = 2 * A_BYTES;
    static_assert(A_BYTES <= 32768 && B_BYTES <= 32768, "slot offsets fit the DS immediate");
    // slot: LDS slot (0 or 1) the tile goes to
    auto store_tile = [&](int slot, const u32x4* a, const u32x4* b) __attribute__((always_inline)) {
      char* sa = smem + slot * A_BYTES;
      char* sb = smem + B_REGION + slot * B_BYTES;
#pragma unroll
      for (int i = 0; i < GA::NIW; ++i) {
        const int jj = wave + NW * i;
        if (GA::TI % NW == 0 || jj < GA::TI)
          *reinterpret_cast<u32x4*>(sa + jj * 1024 + 16 * lane) = a[i];
      }
#pragma unroll
      for (int i = 0; i < GB::NIW; ++i) {
        const int jj = wave + NW * i;
        if (GB::TI % NW == 0 || jj < GB::TI)
          *reinterpret_cast<u32x4*>(sb + jj * 1024 + 16 * lane) = b[i];
      }
    };
    bf16x8 af[2][MF], bf[2][NF];
    // Fragment addresses: per-lane bases (per k-step for k-contiguous tiles,
    // per fragment for output-contiguous ones, which advance by a constant
    // per k-step) plus compile-time offsets. The wave's own row/column offset
    // sits in the base; the fragment index and the slot are immediates.
    // k-contiguous: base_k[ks] + (fr_base[f] - fr_base[0]) * BK * 2
    // output-contiguous: base_f[f] + ks * 16 * ROWS * 2 (+ 4 * ROWS * 2)
    const char* abase[A_KC ? KS : MF];
    const char* bbase[B_KC ? KS : NF];
#pragma unroll
    for (int q = 0; q < (A_KC ? KS : MF); ++q)
      abase[q] = smem + (A_KC ? fa_base[0] * BK * 2 + FA.off[q] : FA.off[q]);
#pragma unroll
    for (int q = 0; q < (B_KC ? KS : NF); ++q)
      bbase[q] = smem + B_REGION + (B_KC ? fb_base[0] * BK * 2 + FB.off[q] : FB.off[q]);
    // compile-time fragment offsets relative to fragment 0 (they depend on
    // the wave only through fr_base[0])
    auto frag_rd = [&](const char* const* base, auto kcc, auto rowsc, int f, int frel, int ks,
                       int slot_off) __attribute__((always_inline)) {
      constexpr bool KC = decltype(kcc)::value;
      constexpr int ROWS = decltype(rowsc)::value;
      if constexpr (KC) {
        return *reinterpret_cast<const bf16x8*>(base[ks] + slot_off + frel * BK * 2);
      } else {
        const char* q = base[f] + slot_off + ks * 16 * ROWS * 2;
        v4s lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) v4s*)(q));
        v4s hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
            (__attribute__((address_space(3))) v4s*)(q + 4 * ROWS * 2));
        v8s r = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
        return __builtin_bit_cast(bf16x8, r);
      }
    };
    auto read_frags = [&](int slot, int ks, int dst) __attribute__((always_inline)) {
#pragma unroll
      for (int mi = 0; mi < MF; ++mi)
        af[dst][mi] = frag_rd(abase, std::integral_constant<bool, A_KC>(),
                              std::integral_constant<int, BM>(), mi, mi * 32, ks, slot * A_BYTES);
#pragma unroll
      for (int ni = 0; ni < NF; ++ni) {
        // fr_base[ni] - fr_base[0]: compile time (paired: gate fragments, then up ones)
        const int frel = PAIRED ? (ni < NF / 2 ? ni * 32 : BN / 2 + (ni - NF / 2) * 32) : ni * 32;
        bf[dst][ni] = frag_rd(bbase, std::integral_constant<bool, B_KC>(),
                              std::integral_constant<int, BN>(), ni, frel, ks, slot * B_BYTES);
      }
    };
    u32x4 ta[GA::NIW], tb[GB::NIW];  // tile 1, prologue only
    if (nk > 0) {
      if (nk0 == 0) switch_plans();
      load_tile(0, ra, rb, true, std::false_type());
      if (1 == nk0) switch_plans();
      load_tile(1, ta, tb, 1 < nk, std::false_type());
      store_tile(0, ra, rb);
      __syncthreads();
      read_frags(0, 0, 0);
    }
    // k-steps of the last tile holding valid k (the rest of it is zeros)
    const int klast = MODE == GROUP_M ? (nk1 > 0 ? p.K[1] - (nk1 - 1) * BK : p.K[0] - (nk0 - 1) * BK)
                                      : krows - (nk0 - 1) * BK;
    const int ns_last = (klast + 15) / 16;
    // One k tile. PAR: the tile's LDS slot when known at compile time (-1:
    // it % 2 at run time). MFMA = false: the wave's rows or columns all lie
    // past the valid ones; it still loads, stores and meets every barrier,
    // but issues no MFMAs and reads no fragments. LAST: the last tile, which
    // stages and loads nothing and leaves its k-step loop after the k-steps
    // that hold valid k (a LoRA segment of rank 16 fills one of a 64-wide
    // tile's four; the rest is zeros); one path with early exits, so the
    // accumulators stay in place. FIRST: tile 1 is stored from the prologue
    // buffer. CLEAN: the load this tile issues (tile it+2) is a whole,
    // in-range tile of the plans already in place.
    auto ktile = [&](int it, auto parc, auto mfmac, auto lastc, auto firstc,
                     auto cleanc) __attribute__((always_inline)) {
      constexpr int PAR = decltype(parc)::value;
      constexpr bool MFMA = decltype(mfmac)::value;
      constexpr bool LAST = decltype(lastc)::value;
      constexpr bool FIRST = decltype(firstc)::value;
      constexpr bool CLEAN = decltype(cleanc)::value;
      const int slot = PAR >= 0 ? PAR : (it & 1);
      if (!CLEAN && it + 2 == nk0) switch_plans();  // the tile loaded here is it+2
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        if constexpr (LAST) {
          if (ks >= ns_last) break;
        }
        const int cur = ks & 1;
        if (ks + 1 < KS) {
          if constexpr (MFMA) read_frags(slot, ks + 1, cur ^ 1);
        } else if (!LAST && it + 1 < nk) {
          // Before the last k-step's MFMAs: every wave has read all of tile
          // it (its slot may be refilled next) and has written tile it+1, so
          // one barrier covers both, and the first fragment reads of tile
          // it+1 overlap this k-step's MFMAs.
          barrier_lds();
          if constexpr (MFMA) read_frags(slot ^ 1, 0, cur ^ 1);
        }
        // tile it+1's slot was last read in tile it-1, before the last barrier
        if (!LAST && ks == 1) {
          // past the last tile this stores the zeros of an out-of-range
          // load into a slot nobody reads again
          if constexpr (FIRST) store_tile(slot ^ 1, ta, tb);
          else store_tile(slot ^ 1, ra, rb);
          const int jn = it + 2;
          if constexpr (CLEAN) load_tile(jn, ra, rb, true, std::true_type());
          else load_tile(min(jn, nk - 1), ra, rb, jn < nk, std::false_type());
        }
        if constexpr (MFMA) {
          // Instruction order within the k-step, by measurement: one LDS read
          // after each MFMA, and in the staging k-step the stores and loads
          // early, two of each after each of the first four MFMAs.
#pragma unroll
          for (int mi = 0; mi < MF; ++mi)
#pragma unroll
            for (int ni = 0; ni < NF; ++ni)
              acc[mi][ni] = mfma32<F16>(bf[cur][ni], af[cur][mi], acc[mi][ni]);
          if (!LAST && ks == 1) {
#pragma unroll
            for (int i = 0; i < MF * NF / 2; ++i) {
              __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // one MFMA
              __builtin_amdgcn_sched_group_barrier(0x200, 2, 0);  // two LDS writes
              __builtin_amdgcn_sched_group_barrier(0x020, 2, 0);  // two buffer loads
            }
#pragma unroll
            for (int i = 0; i < MF * NF / 2; ++i) {
              __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // one MFMA
              __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);  // two LDS reads
            }
          } else {
#pragma unroll
            for (int i = 0; i < MF * NF; ++i) {
              __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // one MFMA
              __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);  // one LDS read
            }
          }
        }
        // Each k-step is a scheduling region of its own: otherwise the
        // scheduler fills the groups above with MFMAs of the next k-step,
        // putting two MFMAs on one accumulator back to back (a dependent
        // 32x32x16 MFMA issues after about 52 cycles instead of 32).
        __builtin_amdgcn_sched_barrier(0);
      }
    };
    // The wave-uniform choice is made once, outside the k loop, so the loop
    // itself has no extra branch.
    auto kloop = [&](auto mfmac) __attribute__((always_inline)) {
      using Yes = std::true_type;
      using No = std::false_type;
      using Rt = std::integral_constant<int, -1>;
      const int nkf = nk - 1;  // full tiles before the last
      // Tiles 1..C are clean: the tile each stages (it + 2) is a whole tile
      // of the main segment (K tail tile excluded).
      const int last_clean = MODE == GROUP_M ? nk0 - 1 - (p.K[0] % BK != 0 ? 1 : 0) : -1;
      const int C = min(nkf - 1, last_clean - 2);
      if (nkf > 0) ktile(0, Rt(), mfmac, No(), Yes(), No());
      int it = 1;
      for (; it + 1 <= C; it += 2) {
        ktile(it, std::integral_constant<int, 1>(), mfmac, No(), No(), Yes());
        ktile(it + 1, std::integral_constant<int, 0>(), mfmac, No(), No(), Yes());
      }
      if (it <= C) {
        ktile(it, std::integral_constant<int, 1>(), mfmac, No(), No(), Yes());
        ++it;
      }
      for (; it < nkf; ++it) ktile(it, Rt(), mfmac, No(), No(), No());
      if (nk > 0) ktile(nkf, Rt(), mfmac, Yes(), No(), No());
    };
    // Waves whose rows all lie past the tile's valid rows, or whose columns
    // all lie past the valid columns, neither read fragments nor multiply.
    const bool live = MODE != GROUP_M ||
                      (wm * WM < rows && (PAIRED ? n_tile * (BN / 2) + wn * (WN / 2) < p.I
                                                 : n0 + wn * WN < p.N));
    if (live) kloop(std::true_type());
    else kloop(std::false_type());
  } else {
    // Gathered reduction rows (GROUP_K, GROUP_KV): the lane offsets of a
    // refill depend on its rows' numbers, so they are formed one iteration
    // ahead (their loads then complete under a k tile of MFMAs instead of
    // delaying the refill's DMA issue).
    constexpr bool gath_a = GATHER_A, gath_b = GATHER_B, gath = GATH != 0;
    uint32_t gvo_a[GA::NIW], gvo_b[GB::NIW];
    // The rows' byte offsets, GT_ROWS at a time from row gw0 on: formed
    // before the first DMA, and again (experts of more than GT_ROWS rows)
    // when a refill passes the window, which then waits for the DMA in flight.
    uint32_t* gt = reinterpret_cast<uint32_t*>(smem + NST * ST + VB_BYTES);
    const int32_t* gt_rows = gath_a ? pa0.view.grow : pb0.view.grow;
    const uint32_t gt_div = static_cast<uint32_t>(gath_a ? pa0.view.gk : pb0.view.gk);
    const uint32_t gt_ld2 = static_cast<uint32_t>(gath_a ? pa0.ld : pb0.ld) * 2u;
    auto gather_window = [&](int w0) __attribute__((always_inline)) {
      __syncthreads();
      for (int i = tid; i < GT_ROWS && w0 + i < krows; i += NW * 64)
        gt[i] = static_cast<uint32_t>(gt_rows[w0 + i]) / gt_div * gt_ld2;
      __syncthreads();
      gw0 = w0;
    };
    if (GT_ROWS > 0 && gath) {
      gather_window(0);
      if (gath_a)
        gtab_a = gt;
      else
        gtab_b = gt;
    }
    auto gather_plan = [&](int j) __attribute__((always_inline)) {
      if (GT_ROWS > 0 && gath && (j + 1) * BK > gw0 + GT_ROWS) gather_window(j * BK);
      if (gath_a) {
#pragma unroll
        for (int i = 0; i < GA::NIW; ++i)
          gvo_a[i] = gather_vo(pa0, j * BK, wave + NW * i, lane, gtab_a, gw0);
      }
      if (gath_b) {
#pragma unroll
        for (int i = 0; i < GB::NIW; ++i)
          gvo_b[i] = gather_vo(pb0, j * BK, wave + NW * i, lane, gtab_b, gw0);
      }
    };
  #pragma unroll
    for (int s = 0; s < NST - 1; ++s)
      if (s < nk) issue(s);
    if (gath && NST - 1 < nk) gather_plan(NST - 1);
    for (int it = 0; it < nk; ++it) {
      // stage `it` must have landed; the DMA-only stages after it may stay in flight
      {
        int ahead = min(NST - 2, nk - 1 - it);
        for (int s = 1; s <= ahead; ++s)
          if (!dma_stage(it + s)) ahead = 0;
        constexpr int PER = GA::MINW + GB::MINW;
        switch (ahead) {
          case 1: wait_vmcnt<PER>(); break;
          case 2: wait_vmcnt<2 * PER>(); break;
          case 3: wait_vmcnt<3 * PER>(); break;
          case 4: wait_vmcnt<4 * PER>(); break;
          default: wait_vmcnt<0>(); break;
        }
      }
      barrier_lds();
      // Stage it+NST-1 is refilled while stage `it` is multiplied: its DMA
      // instructions are spread over the k-steps so that load issue overlaps the
      // MFMAs instead of stalling in-order issue in one burst.
      const int jn = it + NST - 1;
      const bool refill = jn < nk;
      const bool refill_dma = refill && dma_stage(jn);
      if (refill && !refill_dma) issue(jn);  // element-wise fill (rare shapes)
      const bool segn1 = jn >= nk0;
      const int k0n = (segn1 ? jn - nk0 : jn) * BK;
      const Plan<BM, BK, A_KC, NW> PA = segn1 ? pa1 : pa0;
      const Plan<BN, BK, B_KC, NW> PB = segn1 ? pb1 : pb0;
      char* san = smem + (jn % NST) * ST;
      char* sbn = san + A_BYTES;
      const char* sa = smem + (it % NST) * ST;
      const char* sb = sa + A_BYTES;
      constexpr int KS = BK / 16;
      constexpr int NT = GA::NIW + GB::NIW;
      uint32_t gcur_a[GA::NIW], gcur_b[GB::NIW];
#pragma unroll
      for (int i = 0; i < GA::NIW; ++i) gcur_a[i] = gvo_a[i];
#pragma unroll
      for (int i = 0; i < GB::NIW; ++i) gcur_b[i] = gvo_b[i];
      if (gath && jn + 1 < nk) gather_plan(jn + 1);
      // Fragments are double-buffered in registers: the LDS reads of k-step
      // ks+1 are in flight while the MFMAs of k-step ks run.
      bf16x8 af[2][MF], bf[2][NF];
  #pragma unroll
      for (int mi = 0; mi < MF; ++mi) af[0][mi] = read_frag<BM, BK, A_KC, MF>(sa, FA, mi, fa_base[mi], 0);
  #pragma unroll
      for (int ni = 0; ni < NF; ++ni) bf[0][ni] = read_frag<BN, BK, B_KC, NF>(sb, FB, ni, fb_base[ni], 0);
  #pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        const int cur = ks & 1;
        if (ks + 1 < KS) {
  #pragma unroll
          for (int mi = 0; mi < MF; ++mi)
            af[cur ^ 1][mi] = read_frag<BM, BK, A_KC, MF>(sa, FA, mi, fa_base[mi], ks + 1);
  #pragma unroll
          for (int ni = 0; ni < NF; ++ni)
            bf[cur ^ 1][ni] = read_frag<BN, BK, B_KC, NF>(sb, FB, ni, fb_base[ni], ks + 1);
        }
        if (refill_dma) {
  #pragma unroll
          for (int t = ks * NT / KS; t < (ks + 1) * NT / KS; ++t) {
            if (t < GA::NIW) {
              if constexpr (gath_a)
                fill_one<BM, BK, A_KC, NW, false, true>(PA, k0n, san, wave, lane, t, gcur_a[t]);
              else
                fill_one<BM, BK, A_KC, NW, false>(PA, k0n, san, wave, lane, t);
            } else {
              const int tb = t - GA::NIW;
              if constexpr (gath_b)
                fill_one<BN, BK, B_KC, NW, false, true>(PB, k0n, sbn, wave, lane, tb, gcur_b[tb]);
              else
                fill_one<BN, BK, B_KC, NW, false>(PB, k0n, sbn, wave, lane, tb);
            }
          }
        }
  #pragma unroll
        for (int mi = 0; mi < MF; ++mi)
  #pragma unroll
          for (int ni = 0; ni < NF; ++ni)
            acc[mi][ni] = mfma32<F16>(bf[cur][ni], af[cur][mi], acc[mi][ni]);
      }
      if constexpr (MODE == GROUP_KV) {
        // The A stage holds rows it*BK.. of the expert's D as [BK rows][BM
        // features] (output-contiguous layout). One wave per k tile, in turn,
        // multiplies those 32 rows by B over the tile's features and stores
        // the float32 partial; the stage stays valid until the next barrier.
        if (wave == it % NW) {
          f32x16 av;
#pragma unroll
          for (int v = 0; v < 16; ++v) av[v] = 0.f;
          const int kr = lane & 31, hb = lane >> 5;
#pragma unroll
          for (int kk = 0; kk < VKS; ++kk) {
            const int chunk = 2 * kk + hb;  // 8 features 16 kk + 8 hb ..
            const bf16x8 a = *reinterpret_cast<const bf16x8*>(
                sa + kr * BM * 2 + ((chunk ^ nswz<BM>(kr)) << 4));
            av = mfma32<F16>(vbf[kk], a, av);
          }
          // lane holds row kr and columns 8 q + 4 hb + (0..3) for q = 0..3
          const int rowl = it * BK + kr;
          if (rowl < krows) {
            float* vr = p.vp + static_cast<int64_t>(m0 / BM) * p.vp_tstride +
                        (row0 + rowl) * static_cast<int64_t>(p.N);
#pragma unroll
            for (int q = 0; q < 4; ++q) {
              const int j = 8 * q + 4 * hb;
              if (j < p.N)
                *reinterpret_cast<f32x4*>(vr + j) = f32x4{av[4 * q], av[4 * q + 1], av[4 * q + 2], av[4 * q + 3]};
            }
          }
        }
      }
    }

  }

  // ---- Epilogue, staged through LDS. After the final wait no DMA is in
  // flight, so once every wave is past its last fragment read the whole ring
  // is free. Each wave then stages one 32-row slab of its accumulators at a
  // time as float32 and writes the outputs back as whole 16-byte row segments
  // (8 consecutive bf16), which keeps global stores, and the h loads of the
  // SwiGLU backward, coalesced along rows.
  // Accumulator layout: lane holds, for MFMA tile (mi, ni), row lane%32 of the
  // 32-row slab mi and the columns 8*(v/4) + 4*(lane/32) + v%4 of fragment ni.
  __syncthreads();
  constexpr int SLAB = 32 * WN * 4;
  static_assert(NW * SLAB <= NST * ST, "epilogue slab does not fit in the LDS ring");
  char* slab = smem + wave * SLAB;
  const int srow = lane & 31, shalf = lane >> 5;
  const bool out_vec = (reinterpret_cast<uintptr_t>(p.out) & 15) == 0 && (p.ld_out & 7) == 0 &&
                       (p.out_estride & 7) == 0;
  const bool out_vec4 = (reinterpret_cast<uintptr_t>(p.out) & 15) == 0 && (p.ld_out & 3) == 0 &&
                        (p.out_estride & 3) == 0;
  const bool aux_vec = p.aux == nullptr ||
                       ((reinterpret_cast<uintptr_t>(p.aux) & 15) == 0 && (p.ld_aux & 7) == 0);
  // SwiGLU backward: the h segments a slab needs are loaded while the previous
  // slab is finished, so one load latency per tile is exposed rather than one
  // per slab (the epilogue reads h [rows, 2I] and writes dH of the same size).
  // (wave tiles up to 64 wide: two slabs of h take 64 VGPRs; wider ones load per slab)
  constexpr bool HPRE = MODE == GROUP_M && EPI == EPI_SWIGLU_BWD && !PAIRED && WN <= 64;
  constexpr int HSEGS = WN / 8, HRPP = 64 / HSEGS, HPASS = 32 / HRPP;
  u32x4 hpre[2][HPASS][2];
  auto hfetch = [&](int mi, u32x4 (&hb)[HPASS][2]) {
    const int mb = wm * WM + mi * 32;
#pragma unroll
    for (int pass = 0; pass < HPASS; ++pass) {
      const int m_local = mb + pass * HRPP + lane / HSEGS;
      const int col = n0 + wn * WN + 8 * (lane % HSEGS);
      if (m_local < rows && col < p.N) {  // N = I, a multiple of 8
        const bf16_t* hr = static_cast<const bf16_t*>(p.aux) + (row0 + m_local) * p.ld_aux;
        hb[pass][0] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(hr + col));
        hb[pass][1] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(hr + p.I + col));
      }
    }
  };
  if constexpr (HPRE) hfetch(0, hpre[0]);
#pragma unroll
  for (int mi = 0; mi < MF; ++mi) {
    if constexpr (HPRE) {
      if (mi + 1 < MF) hfetch(mi + 1, hpre[(mi + 1) & 1]);
    }
    if (mi) wave_lds_sync();  // previous slab fully read
#pragma unroll
    for (int ni = 0; ni < NF; ++ni)
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        f32x4 v;
#pragma unroll
        for (int j = 0; j < 4; ++j) v[j] = acc[mi][ni][4 * q + j];
        *reinterpret_cast<f32x4*>(slab + slab_off<WN>(srow, ni * 8 + 2 * q + shalf)) = v;
      }
    wave_lds_sync();
    const int mbase = wm * WM + mi * 32;  // first tile row of this slab
    if (PAIRED) {
      // slab columns [0, WN/2) are gate features, [WN/2, WN) the matching up features
      constexpr int SEGS = WN / 16, RPP = 64 / SEGS;
#pragma unroll
      for (int pass = 0; pass < 32 / RPP; ++pass) {
        const int r = pass * RPP + lane / SEGS, s = lane % SEGS;
        const int m_local = mbase + r;
        const int f = n_tile * (BN / 2) + wn * (WN / 2) + 8 * s;
        float g[8], u[8], a[8];
        read8<WN>(slab, r, 2 * s, g);
        read8<WN>(slab, r, WN / 8 + 2 * s, u);
        if (m_local < rows && f < p.I) {  // I is a multiple of 8
#pragma unroll
          for (int j = 0; j < 8; ++j) a[j] = swiglu(g[j], u[j]);
          const int64_t row = row0 + m_local;
          bf16_t* hr = static_cast<bf16_t*>(p.out) + row * p.ld_out;
          store8<F16>(hr + f, g);
          store8<F16>(hr + p.I + f, u);
          store8<F16>(static_cast<bf16_t*>(p.out2) + row * p.ld_out2 + f, a);
        }
      }
    } else {
      constexpr int SEGS = WN / 8, RPP = 64 / SEGS;
#pragma unroll
      for (int pass = 0; pass < 32 / RPP; ++pass) {
        const int r = pass * RPP + lane / SEGS, s = lane % SEGS;
        const int m_local = mbase + r;
        const int col = n0 + wn * WN + 8 * s;
        float v[8];
        read8_interleaved<WN>(slab, r, s, v);
        if (MODE == GROUP_M && EPI == EPI_SWIGLU_BWD) {
          // every lane stays to the end: the dw partial is summed over the
          // SEGS lanes that hold one row
          const int64_t row = row0 + m_local;
          float part = 0.f;
          if (m_local < rows && col < p.N) {  // N = I, a multiple of 8
            float g[8], u[8], dg[8], du[8];
            if constexpr (HPRE) {
              unpack8<F16>(hpre[mi & 1][pass][0], g);
              unpack8<F16>(hpre[mi & 1][pass][1], u);
            } else {
              const bf16_t* hr = static_cast<const bf16_t*>(p.aux) + row * p.ld_aux;
              load8<F16>(hr + col, g);
              load8<F16>(hr + p.I + col, u);
            }
            const float wr = p.roww ? p.roww[row] : 1.0f;
#pragma unroll
            for (int j = 0; j < 8; ++j)
              part += v[j] * swiglu_bwd_act(g[j], u[j], wr * v[j], dg[j], du[j]);
            bf16_t* dr = static_cast<bf16_t*>(p.out) + row * p.ld_out;
            store8<F16>(dr + col, dg);
            store8<F16>(dr + p.I + col, du);
          }
          if (p.dwp) {
#pragma unroll
            for (int off = SEGS / 2; off >= 1; off >>= 1) part += __shfl_xor(part, off, kWave);
            if (s == 0 && m_local < rows)
              p.dwp[row * p.dwp_slots + n_tile * WAVES_N + wn] = part;
          }
          continue;
        }
        if (m_local >= rows) continue;
        if (EPI == EPI_STORE_F32) {
          // GROUP_M: router logits; GROUP_K: split-K partial weight gradients
          float* rp = MODE == GROUP_M
                          ? static_cast<float*>(p.out) + (row0 + m_local) * p.ld_out
                          : static_cast<float*>(p.out) + static_cast<int64_t>(e) * p.out_estride +
                                static_cast<int64_t>(m0 + m_local) * p.ld_out;
          if (out_vec4 && col + 8 <= p.N) {
            float4* q = reinterpret_cast<float4*>(rp + col);
            q[0] = make_float4(v[0] * p.scale, v[1] * p.scale, v[2] * p.scale, v[3] * p.scale);
            q[1] = make_float4(v[4] * p.scale, v[5] * p.scale, v[6] * p.scale, v[7] * p.scale);
          } else {
#pragma unroll
            for (int j = 0; j < 8; ++j)
              if (col + j < p.N) rp[col + j] = v[j] * p.scale;
          }
        } else {
#pragma unroll
          for (int j = 0; j < 8; ++j) v[j] *= p.scale;
          // GROUP_M: an expert's row; GROUP_K: feature row m0 + m_local of expert e's gradient
          bf16_t* rp = MODE == GROUP_M
                           ? static_cast<bf16_t*>(p.out) + (row0 + m_local) * p.ld_out
                           : static_cast<bf16_t*>(p.out) + static_cast<int64_t>(e) * p.out_estride +
                                 static_cast<int64_t>(m0 + m_local) * p.ld_out;
          // EPI_ADD source row: aux (merged export) or the output row itself
          const bf16_t* sp = EPI == EPI_ADD && p.aux
                                 ? static_cast<const bf16_t*>(p.aux) + (row0 + m_local) * p.ld_aux
                                 : rp;
          if (out_vec && col + 8 <= p.N && (EPI != EPI_ADD || aux_vec)) {
            if (EPI == EPI_ADD) {
              float o[8];
              load8<F16>(sp + col, o);
#pragma unroll
              for (int j = 0; j < 8; ++j) v[j] += o[j];
            }
            store8<F16>(rp + col, v);
          } else {
#pragma unroll
            for (int j = 0; j < 8; ++j)
              if (col + j < p.N)
                rp[col + j] = f32_to_h16<F16>(EPI == EPI_ADD ? v[j] + h16_to_f32<F16>(sp[col + j]) : v[j]);
          }
        }
      }
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
      if (A.rows) {
        va.base = static_cast<const float*>(A.ptr);
        va.grow = A.rows + row0;
        va.gk = A.rows_div;
      }
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
      if (A.rows) {
        va.base = static_cast<const float*>(A.ptr) + m0;
        va.grow = A.rows + row0;
        va.gk = A.rows_div;
      }
      vb.base = static_cast<const float*>(B.ptr) + row0 * B.ld + n0;
      vb.mn_lim = p.N - n0;
      if (B.rows) {
        vb.base = static_cast<const float*>(B.ptr) + n0;
        vb.grow = B.rows + row0;
        vb.gk = B.rows_div;
      }
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
  if constexpr (!PAIRED && MODE == GROUP_M && EPI == EPI_SWIGLU_BWD) {
    // SwiGLU backward with optional row weights and dw partials (one slot per
    // N tile, summed over the 16 threads of a row: consecutive lanes)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int m_local = ty * 4 + i;
      const int64_t row = row0 + m_local;
      float part = 0.f;
      if (m_local < rows) {
        const float* hr = static_cast<const float*>(p.aux) + row * p.ld_aux;
        float* dr = static_cast<float*>(p.out) + row * p.ld_out;
        const float wr = p.roww ? p.roww[row] : 1.0f;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const int col = n0 + tx * 4 + j;
          if (col < p.N) {
            const float g = hr[col], u = hr[p.I + col];
            float dg, du;
            part += acc[i][j] * swiglu_bwd_act(g, u, wr * acc[i][j], dg, du);
            dr[col] = dg;
            dr[p.I + col] = du;
          }
        }
      }
      if (p.dwp) {
#pragma unroll
        for (int off = 8; off >= 1; off >>= 1) part += __shfl_xor(part, off, kWave);
        if (tx == 0 && m_local < rows) p.dwp[row * p.dwp_slots + n_tile] = part;
      }
    }
    return;
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
// One block of 1024 threads (E <= 1024). Two lists in one launch, for two tile
// heights: M tiles of `bm` rows per expert, in expert order, with their raster
// groups (group_tile); empty experts get none.
__global__ __launch_bounds__(1024) void tiles_kernel(const int32_t* __restrict__ offsets, int E,
                                                     int bm0, int4* __restrict__ tiles0,
                                                     int32_t* __restrict__ ntiles0, int bm1,
                                                     int4* __restrict__ tiles1,
                                                     int32_t* __restrict__ ntiles1) {
  __shared__ int wsum[2][1024 / kWave];
  const int lane = threadIdx.x & (kWave - 1), wave = threadIdx.x / kWave;
  const int e = threadIdx.x;
  int lo = 0, cnt = 0;
  if (e < E) {
    lo = offsets[e];
    cnt = offsets[e + 1] - lo;
  }
#pragma unroll
  for (int l = 0; l < 2; ++l) {
    const int bm = l ? bm1 : bm0;
    int4* tiles = l ? tiles1 : tiles0;
    const int nt = (cnt + bm - 1) / bm;
    int incl = nt;
#pragma unroll
    for (int off = 1; off < kWave; off <<= 1) {
      int o = __shfl_up(incl, off, kWave);
      if (lane >= off) incl += o;
    }
    if (lane == kWave - 1) wsum[l][wave] = incl;
    __syncthreads();
    int base = 0, total = 0;
    for (int w = 0; w < 1024 / kWave; ++w) {
      if (w < wave) base += wsum[l][w];
      total += wsum[l][w];
    }
    base += incl - nt;
    for (int i = 0; i < nt; ++i) {
      const int r = i * bm;
      const int g0 = i / kTileGroup * kTileGroup;
      const int grp = (base + g0) * 16 + min(kTileGroup, nt - g0);
      tiles[base + i] = make_int4(e, lo + r, min(bm, cnt - r), grp);
    }
    if (threadIdx.x == 0) *(l ? ntiles1 : ntiles0) = total;
  }
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
  o.rows = nullptr;
  o.rows_div = 1;
  o.rows_bytes = 0;
  return o;
}

Opnd none() { return Opnd{nullptr, 0, 0, 1, 0, nullptr, 1, 0}; }

inline int esz_of(const ExpertDims& d) { return d.dtype == MOE_F32 ? 4 : 2; }

// The layer input [rows, ld] as an operand: x_perm as it is, or x in token
// order read through sorted_pair.
Opnd opnd_x(const XRows& x, int64_t ld, int kcontig, int esz) {
  Opnd o = opnd(x.ptr, 0, ld, kcontig, true);
  if (x.rows) {
    o.rows = x.rows;
    o.rows_div = x.k;
    o.rows_bytes = static_cast<int64_t>(x.T) * ld * esz;
  }
  return o;
}

// Tile list capacity for `bm`-row tiles.
inline int64_t tile_cap(int64_t N, int E, int bm) { return (N + bm - 1) / bm + E + 1; }

// Two device-built tile lists: `small` (the LoRA side products and the
// float32 kernels) and `big` (the four expert GEMMs; its tile height depends
// on the tile variant).
struct TileList {
  int4* tiles;
  int32_t* ntiles;
  int bm;
};

struct WsLayout {
  TileList small, big;
  size_t bytes;
};

inline int small_rows(int dtype) { return dtype != MOE_F32 ? 128 : 64; }
// 256-row tiles for the register-staged kernel, whose LoRA segment (K = r)
// must come in 16-byte pieces.
inline int big_rows(const ExpertDims& d) {
  if (d.dtype == MOE_F32) return 64;
  return d.r % 8 == 0 ? 256 : 128;
}

WsLayout tile_ws(void* ws, const ExpertDims& d) {
  WsLayout L;
  char* p = static_cast<char*>(ws);
  size_t off = 0;
  auto list = [&](int bm) {
    TileList t;
    t.bm = bm;
    t.tiles = reinterpret_cast<int4*>(p + off);
    off += align_up(static_cast<size_t>(tile_cap(d.N, d.E, bm)) * sizeof(int4));
    t.ntiles = reinterpret_cast<int32_t*>(p + off);
    off += kAlign;
    return t;
  };
  L.small = list(small_rows(d.dtype));
  L.big = list(big_rows(d));
  L.bytes = off;
  return L;
}

inline hipError_t build_tiles(const WsLayout& L, const int32_t* offsets, int E, hipStream_t s) {
  hipLaunchKernelGGL(tiles_kernel, dim3(1), dim3(1024), 0, s, offsets, E, L.small.bm,
                     L.small.tiles, L.small.ntiles, L.big.bm, L.big.tiles, L.big.ntiles);
  return hipGetLastError();
}

template <typename K>
hipError_t launch(K kern, int grid, const GemmArgs& a, hipStream_t s, int threads = 256) {
  if (grid <= 0) return hipSuccess;
  hipLaunchKernelGGL(kern, dim3(grid), dim3(threads), 0, s, a);
  return hipGetLastError();
}

// The 16-bit GEMM instantiation for a layer dtype (MOE_BF16 or MOE_F16); the
// arguments are the tile parameters of gemm16 after F16, VST last.
#define GEMM16(dtype, ...) \
  ((dtype) == MOE_F16 ? gemm16<true, __VA_ARGS__> : gemm16<false, __VA_ARGS__>)

// Tiles of the four expert GEMMs, chosen by measurement on MI355X:
//  - 256 x 256, eight waves of 128 x 64, BK 64, two LDS slots (128 KB),
//    operands staged through VGPRs (one k tile in flight per wave): the
//    default. A wave issues buffer->LDS DMA at about a quarter of the rate it
//    issues buffer loads into VGPRs, so register staging keeps the MFMAs fed
//    with fewer bytes in flight; 256-row tiles also halve the L2 traffic per
//    MFMA relative to 128 x 256.
//  - 256 x 256 with buffer->LDS DMA fills (128 x 128 per wave, BK 32, three
//    stages) when an operand cannot be read in 16-byte pieces (a pointer that
//    is not 16-byte aligned): the DMA fill falls back to element-wise loads.
//  - 128 x 256, four waves, buffer->LDS DMA, BK 32, three stages, two blocks
//    per CU: ranks that are not a multiple of 8 (the LoRA segment, K = r,
//    then takes element-wise fills).
inline bool all_vec(const GemmArgs& a) {
  return a.a[0].vec && a.b[0].vec && (a.K[1] == 0 || (a.a[1].vec && a.b[1].vec));
}

// Wave columns per N tile of the kernel launch_big runs (the dw partial
// slots of a SwiGLU-backward launch): 256 / 64 for the register-staged
// kernel, 256 / 128 for the other two.
inline int big_waves_n(const GemmArgs& a, int bm) { return bm == 256 && all_vec(a) ? 4 : 2; }

template <int MODE, int EPI, bool PAIRED, bool A_KC, bool B_KC>
hipError_t launch_big(int grid, const GemmArgs& a, hipStream_t s, int bm) {
  if (bm == 256) {
    if (!all_vec(a))
      return launch(GEMM16(a.dtype, 256, 256, 128, 128, 32, 3, 1, MODE, EPI, PAIRED, A_KC, B_KC, 0), grid, a, s);
    return launch(GEMM16(a.dtype, 256, 256, 128, 64, 64, 2, 1, MODE, EPI, PAIRED, A_KC, B_KC, 1), grid, a, s, 512);
  }
  return launch(GEMM16(a.dtype, 128, 256, 64, 128, 32, 3, 2, MODE, EPI, PAIRED, A_KC, B_KC, 0), grid, a, s);
}

// M-tile grid bound for GROUP_M launches over a tile list (excess blocks exit at once).
inline int gm_grid(const ExpertDims& d, const TileList& t, int ntn) {
  return static_cast<int>(tile_cap(d.N, d.E, t.bm) * ntn);
}

GemmArgs base_args(const ExpertDims& d, const int32_t* offsets, const TileList& t) {
  GemmArgs a{};
  a.a[1] = none();
  a.b[1] = none();
  a.E = d.E;
  a.offsets = offsets;
  a.tiles = t.tiles;
  a.ntiles = t.ntiles;
  a.I = d.I;
  a.scale = 1.0f;
  a.dtype = d.dtype;
  return a;
}

// out[rows, r] = scale * A[rows, K] * L_e (L_e is [r, K] when l_kcontig, else [K, r]).
hipError_t side_product(const ExpertDims& d, const int32_t* offsets, const WsLayout& L,
                        const Opnd& A, int K, const void* Lw, int64_t l_estride, int l_kcontig,
                        void* out, hipStream_t s) {
  const TileList& t = L.small;
  GemmArgs a = base_args(d, offsets, t);
  const bool r_vec = d.r % 8 == 0;
  a.a[0] = A;
  a.b[0] = l_kcontig ? opnd(Lw, l_estride, K, 1, true) : opnd(Lw, l_estride, d.r, 0, r_vec);
  a.K[0] = K;
  a.K[1] = 0;
  a.N = d.r;
  a.out = out;
  a.ld_out = d.r;
  a.scale = d.scale;
  if (d.dtype != MOE_F32) {
    a.ntn = 1;
    if (l_kcontig) {
      if (d.r <= 32)
        return launch(GEMM16(a.dtype, 128, 32, 32, 32, 64, 3, 2, GROUP_M, EPI_STORE, false, true, true, 0),
                      gm_grid(d, t, 1), a, s);
      return launch(GEMM16(a.dtype, 128, 64, 32, 64, 64, 3, 2, GROUP_M, EPI_STORE, false, true, true, 0),
                    gm_grid(d, t, 1), a, s);
    }
    if (d.r <= 32)
      return launch(GEMM16(a.dtype, 128, 32, 32, 32, 64, 3, 2, GROUP_M, EPI_STORE, false, true, false, 0),
                    gm_grid(d, t, 1), a, s);
    return launch(GEMM16(a.dtype, 128, 64, 32, 64, 64, 3, 2, GROUP_M, EPI_STORE, false, true, false, 0),
                  gm_grid(d, t, 1), a, s);
  }
  a.ntn = ceil_div(d.r, 64);
  return launch(gemm_f32<GROUP_M, EPI_STORE, false>, gm_grid(d, t, a.ntn), a, s);
}

// ---- weight gradients: out_e[P, Q] = sum over the expert's rows n of L[n, P] R[n, Q]
// (L: [rows, P], R: [rows, Q]). One workgroup owns an output tile and runs
// over all the expert's rows, so no atomics are needed and the result does not
// depend on scheduling. When the experts are too few to give every CU a tile
// (a shared expert is one expert over all T tokens), each expert's rows are
// cut into S contiguous chunks that act as experts of their own, every chunk
// writes a float32 partial into the workspace, and a second kernel sums the S
// partials of each expert in chunk order (still deterministic).

// Tiles per expert of the kernel weight_grad picks for [P, Q].
int wgrad_tiles(const ExpertDims& d, int P, int Q) {
  if (d.dtype == MOE_F32) return ceil_div(P, 64) * ceil_div(Q, 64);
  if (Q <= 64 && P > 64) return ceil_div(P, 256);
  if (P >= 256 && Q >= 256) return ceil_div(P, 128) * ceil_div(Q, 256);
  return (P <= 32 ? 1 : ceil_div(P, 64)) * ceil_div(Q, 256);
}

// Row chunks per expert: enough to reach ~512 workgroups when fewer than 256
// would run, never chunks of fewer than 256 rows on average, and only for the
// LoRA gradients of rank <= 32 (the full fine-tuning gradients have tiles
// enough and would need large partials; higher ranks are rare).
int wgrad_splits(const ExpertDims& d, int P, int Q) {
  if (std::min(P, Q) > 32) return 1;
  const int64_t blocks = static_cast<int64_t>(d.E) * wgrad_tiles(d, P, Q);
  if (blocks >= 256) return 1;
  const int64_t by_rows = static_cast<int64_t>(d.N) / (static_cast<int64_t>(d.E) * 256);
  const int64_t want = (512 + blocks - 1) / blocks;
  return static_cast<int>(std::max<int64_t>(1, std::min<int64_t>({want, by_rows, 64})));
}

// Workspace for the split path of one [P, Q] gradient: chunk offsets, then partials.
size_t wgrad_split_bytes(const ExpertDims& d, int P, int Q) {
  const int S = wgrad_splits(d, P, Q);
  if (S <= 1) return 0;
  const int64_t G = static_cast<int64_t>(d.E) * S;
  return align_up(static_cast<size_t>(G + 1) * 4) + align_up(static_cast<size_t>(G) * P * Q * 4);
}

// The largest split workspace over the four LoRA gradients of the backward.
size_t lora_wgrad_split_bytes(const ExpertDims& d) {
  const int H = d.H, I = d.I, r = d.r;
  return std::max({wgrad_split_bytes(d, H, r), wgrad_split_bytes(d, r, I),
                   wgrad_split_bytes(d, 2 * I, r), wgrad_split_bytes(d, r, H)});
}

// Chunk c of expert e covers rows [off[e] + cnt_e c / S, off[e] + cnt_e (c + 1) / S).
__global__ void split_offsets_kernel(const int32_t* __restrict__ off, int E, int S,
                                     int32_t* __restrict__ voff) {
  for (int i = threadIdx.x; i < E * S; i += blockDim.x) {
    const int e = i / S, c = i - e * S;
    const int64_t cnt = off[e + 1] - off[e];
    voff[i] = off[e] + static_cast<int32_t>(cnt * c / S);
  }
  if (threadIdx.x == 0) voff[E * S] = off[E];
}

template <typename Elem>
__global__ __launch_bounds__(256) void reduce_splits_kernel(const float* __restrict__ part,
                                                            Elem* __restrict__ out, int S,
                                                            int64_t PQ, int64_t total) {
  const int64_t i = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
  if (i >= total) return;
  const int64_t e = i / PQ, q = i - e * PQ;
  const float* p = part + e * S * PQ + q;
  float acc = 0.f;
  for (int c = 0; c < S; ++c) acc += p[c * PQ];
  out[i] = from_f32<Elem>(acc);
}

// One weight-gradient tile shape (BK 32, three stages, two blocks per CU): the
// instantiation that reads A's rows (GA) or B's rows (GB) through their row
// list when that operand has one. Shapes without that instantiation refuse a
// row list, as does a launch with both.
template <int BM, int BN, int WM, int WN, int MODE, int EPI, bool GA, bool GB>
hipError_t launch_wg(const GemmArgs& a, int grid, hipStream_t s) {
  const bool ra = a.a[0].rows != nullptr, rb = a.b[0].rows != nullptr;
  if (ra && rb) return hipErrorInvalidValue;
  if (ra) {
    if constexpr (GA)
      return launch(GEMM16(a.dtype, BM, BN, WM, WN, 32, 3, 2, MODE, EPI, false, false, false, 0, 1),
                    grid, a, s);
    return hipErrorInvalidValue;
  }
  if (rb) {
    if constexpr (GB)
      return launch(GEMM16(a.dtype, BM, BN, WM, WN, 32, 3, 2, MODE, EPI, false, false, false, 0, 2),
                    grid, a, s);
    return hipErrorInvalidValue;
  }
  return launch(GEMM16(a.dtype, BM, BN, WM, WN, 32, 3, 2, MODE, EPI, false, false, false, 0),
                grid, a, s);
}

template <int EPI>
hipError_t weight_grad_launch(const ExpertDims& d, GemmArgs& a, int E, int P, int Q,
                              hipStream_t s) {
  if (a.vp) {  // [big, r <= 32] with side-product partials (checked by the caller)
    a.ntn = 1;
    a.ntm = ceil_div(P, 256);
    return launch_wg<256, 32, 64, 32, GROUP_KV, EPI, true, false>(a, E * a.ntm, s);
  }
  if (d.dtype != MOE_F32) {
    // Split partials (EPI_STORE_F32) only come from gradients with a side of
    // at most 32 (wgrad_splits): the other tile shapes exist for EPI_STORE only.
    constexpr bool WIDE = EPI == EPI_STORE;
    if (Q <= 64 && P > 64) {  // [big, r]
      a.ntn = 1;
      a.ntm = ceil_div(P, 256);
      if (Q <= 32) return launch_wg<256, 32, 64, 32, GROUP_K, EPI, true, false>(a, E * a.ntm, s);
      if constexpr (WIDE)
        return launch_wg<256, 64, 64, 64, GROUP_K, EPI, true, false>(a, E * a.ntm, s);
      return hipErrorInvalidValue;
    }
    if (P >= 256 && Q >= 256) {  // [big, big]: full fine-tuning weight gradients
      if constexpr (WIDE) {
        a.ntm = ceil_div(P, 128);
        a.ntn = ceil_div(Q, 256);
        return launch_wg<128, 256, 64, 128, GROUP_K, EPI, false, true>(a, E * a.ntm * a.ntn, s);
      }
      return hipErrorInvalidValue;
    }
    // [r, big] (or both small)
    a.ntn = ceil_div(Q, 256);
    if (P <= 32) {
      a.ntm = 1;
      return launch_wg<32, 256, 32, 64, GROUP_K, EPI, false, true>(a, E * a.ntn, s);
    }
    if constexpr (WIDE) {
      a.ntm = ceil_div(P, 64);
      return launch_wg<64, 256, 64, 64, GROUP_K, EPI, true, true>(a, E * a.ntm * a.ntn, s);
    }
    return hipErrorInvalidValue;
  }
  a.ntm = ceil_div(P, 64);
  a.ntn = ceil_div(Q, 64);
  return launch(gemm_f32<GROUP_K, EPI_STORE, false>, E * a.ntm * a.ntn, a, s);
}

#define MOE_TRY_WG(x)                   \
  do {                                  \
    hipError_t err_ = (x);              \
    if (err_ != hipSuccess) return err_; \
  } while (0)

// Side product fused into a LoRA B gradient (see GROUP_KV): alongside
// dB = D^T U it forms V = scale * D Bm with Bm per expert [P, Q].
struct SideOut {
  const void* bm = nullptr;   // [E][P][Q]
  void* out = nullptr;        // V [N, Q] in the layer dtype
  float* part = nullptr;      // ceil(P / 256) x N x Q float32 partials
  const float* roww = nullptr;  // optional: also out_w[n] = roww[n] V[n] (one rounding)
  void* out_w = nullptr;
};

// The fused path covers 16-bit layers, Q = r <= 32 with rows of 16 bytes.
// The partials cost ceil(P / 256) x Q float32 per row each way; past 2 KB a
// row (512 values: DeepSeek-V3's dB_d, 28 tiles at r = 32) reading D a second
// time in a plain side-product GEMM was faster on MI355X (0.45 against
// 0.53 ms), at 2 KB the two were even (DeepSeek-V3's dB_gu), below it fusing
// wins (gpt-oss-20b's dB_gu, 1.5 KB: 0.11 against 0.17 ms).
inline bool side_fusable(const ExpertDims& d, int P, int Q) {
  return d.dtype != MOE_F32 && Q <= 32 && Q % 8 == 0 && P % 8 == 0 && P > 64 &&
         ceil_div(P, 256) * Q <= 512;
}

inline size_t side_part_bytes(const ExpertDims& d) {
  int P = 0;
  for (const int p : {d.H, 2 * d.I})
    if (side_fusable(d, p, d.r)) P = std::max(P, p);
  return static_cast<size_t>(ceil_div(P, 256)) * d.N * d.r * 4;
}

// V[i] = scale * sum over tiles t (in order) of part[t][i]; with roww, also
// out_w[i] = roww[i / Q] * V[i] (from the float32 sum, one rounding).
template <typename Elem>
__global__ __launch_bounds__(256) void side_sum_kernel(const float* __restrict__ part, int tiles,
                                                       int64_t tstride, float scale,
                                                       Elem* __restrict__ out,
                                                       const float* __restrict__ roww, int Q,
                                                       Elem* __restrict__ out_w) {
  const int64_t i = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
  if (i >= tstride) return;
  float acc = 0.f;
  for (int t = 0; t < tiles; ++t) acc += part[t * tstride + i];
  out[i] = from_f32<Elem>(acc * scale);
  if (roww) out_w[i] = from_f32<Elem>(roww[i / Q] * (acc * scale));
}

// dst[n][c] = w[n] * src[n][c] over rows x cols (dst may be src), one rounding.
// VEC (16-bit, cols % 8 == 0, both 16-byte aligned: the dY rows of full
// fine-tuning) one 16-byte piece per thread; otherwise (float32 rows, and the
// [N, r] side products when r % 8 != 0) one element per thread.
template <typename Elem, bool VEC>
__global__ __launch_bounds__(256) void scale_rows_kernel(const Elem* src, const float* __restrict__ w,
                                                         int64_t total, int cols, Elem* dst) {
  const int64_t i = (static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x) * (VEC ? 8 : 1);
  if (i >= total) return;
  const float wr = w[i / cols];
  if constexpr (VEC) {
    u32x4 v = *reinterpret_cast<const u32x4*>(src + i);
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      const uint16_t lo = static_cast<uint16_t>(v[t] & 0xffffu), hi = static_cast<uint16_t>(v[t] >> 16);
      const float a = wr * to_f32<Elem>(__builtin_bit_cast(Elem, lo));
      const float b = wr * to_f32<Elem>(__builtin_bit_cast(Elem, hi));
      v[t] = static_cast<uint32_t>(__builtin_bit_cast(uint16_t, from_f32<Elem>(a))) |
             (static_cast<uint32_t>(__builtin_bit_cast(uint16_t, from_f32<Elem>(b))) << 16);
    }
    *reinterpret_cast<u32x4*>(dst + i) = v;
  } else {
    dst[i] = from_f32<Elem>(wr * to_f32<Elem>(src[i]));
  }
}

hipError_t scale_rows(int dtype, const void* src, const float* w, int64_t rows, int cols,
                      void* dst, hipStream_t s) {
  const int64_t total = rows * cols;
  if (total <= 0) return hipSuccess;
  const bool vec = dtype != MOE_F32 && cols % 8 == 0 && aligned16(src) && aligned16(dst);
  const dim3 grid(static_cast<unsigned>((total / (vec ? 8 : 1) + 255) / 256));
  if (dtype == MOE_BF16) {
    auto k = vec ? scale_rows_kernel<bf16_t, true> : scale_rows_kernel<bf16_t, false>;
    hipLaunchKernelGGL(k, grid, dim3(256), 0, s, static_cast<const bf16_t*>(src), w, total, cols,
                       static_cast<bf16_t*>(dst));
  } else if (dtype == MOE_F16) {
    auto k = vec ? scale_rows_kernel<f16_t, true> : scale_rows_kernel<f16_t, false>;
    hipLaunchKernelGGL(k, grid, dim3(256), 0, s, static_cast<const f16_t*>(src), w, total, cols,
                       static_cast<f16_t*>(dst));
  } else {
    auto k = scale_rows_kernel<float, false>;
    hipLaunchKernelGGL(k, grid, dim3(256), 0, s, static_cast<const float*>(src), w, total, cols,
                       static_cast<float*>(dst));
  }
  return hipGetLastError();
}

// split_ws: at least wgrad_split_bytes(d, P, Q) bytes (unused when that is 0),
// or null: then the rows are never split (one workgroup per output tile runs
// over all of an expert's rows), whatever wgrad_splits would choose.
// side (optional, side_fusable only): also form V = scale D Bm.
hipError_t weight_grad(const ExpertDims& d, const int32_t* offsets, const void* Lm, int P,
                       const void* Rm, int Q, void* out, hipStream_t s, void* split_ws,
                       const SideOut* side = nullptr, const XRows* rx = nullptr,
                       const XRows* lx = nullptr) {
  if (lx && rx) return hipErrorInvalidValue;  // at most one operand's rows are gathered
  GemmArgs a{};
  a.vsplit = 1;
  if (side) {
    a.vb = side->bm;
    a.vb_estride = static_cast<int64_t>(P) * Q;
    a.vp = side->part;
    a.vp_tstride = d.N * Q;
  }
  a.a[1] = none();
  a.b[1] = none();
  a.M = P;
  a.N = Q;
  a.scale = 1.0f;
  a.dtype = d.dtype;
  a.out_estride = static_cast<int64_t>(P) * Q;
  a.ld_out = Q;
  a.a[0] = lx ? opnd_x(*lx, P, 0, esz_of(d)) : opnd(Lm, 0, P, 0, P % 8 == 0);
  a.b[0] = rx ? opnd_x(*rx, Q, 0, esz_of(d)) : opnd(Rm, 0, Q, 0, Q % 8 == 0);
  const int S = split_ws ? wgrad_splits(d, P, Q) : 1;
  auto side_sum = [&]() -> hipError_t {
    if (!side) return hipSuccess;
    const int tiles = ceil_div(P, 256);
    const int64_t n = d.N * Q;
    const dim3 grid(static_cast<unsigned>((n + 255) / 256));
    if (d.dtype == MOE_BF16)
      hipLaunchKernelGGL(side_sum_kernel<bf16_t>, grid, dim3(256), 0, s, side->part, tiles, n,
                         d.scale, static_cast<bf16_t*>(side->out), side->roww, Q,
                         static_cast<bf16_t*>(side->out_w));
    else
      hipLaunchKernelGGL(side_sum_kernel<f16_t>, grid, dim3(256), 0, s, side->part, tiles, n,
                         d.scale, static_cast<f16_t*>(side->out), side->roww, Q,
                         static_cast<f16_t*>(side->out_w));
    return hipGetLastError();
  };
  if (S <= 1) {
    a.E = d.E;
    a.offsets = offsets;
    a.out = out;
    MOE_TRY_WG(weight_grad_launch<EPI_STORE>(d, a, d.E, P, Q, s));
    return side_sum();
  }
  const int G = d.E * S;
  a.vsplit = S;
  int32_t* voff = static_cast<int32_t*>(split_ws);
  float* part = reinterpret_cast<float*>(static_cast<char*>(split_ws) +
                                         align_up(static_cast<size_t>(G + 1) * 4));
  hipLaunchKernelGGL(split_offsets_kernel, dim3(1), dim3(256), 0, s, offsets, d.E, S, voff);
  a.E = G;
  a.offsets = voff;
  a.out = part;
  hipError_t e = weight_grad_launch<EPI_STORE_F32>(d, a, G, P, Q, s);
  if (e != hipSuccess) return e;
  const int64_t PQ = static_cast<int64_t>(P) * Q, total = static_cast<int64_t>(d.E) * PQ;
  const dim3 grid(static_cast<unsigned>((total + 255) / 256));
  if (d.dtype == MOE_BF16)
    hipLaunchKernelGGL(reduce_splits_kernel<bf16_t>, grid, dim3(256), 0, s, part,
                       static_cast<bf16_t*>(out), S, PQ, total);
  else if (d.dtype == MOE_F16)
    hipLaunchKernelGGL(reduce_splits_kernel<f16_t>, grid, dim3(256), 0, s, part,
                       static_cast<f16_t*>(out), S, PQ, total);
  else
    hipLaunchKernelGGL(reduce_splits_kernel<float>, grid, dim3(256), 0, s, part,
                       static_cast<float*>(out), S, PQ, total);
  MOE_TRY_WG(hipGetLastError());
  return side_sum();
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

namespace {

// dw partial slots per row of the down backward (the combine backward folded
// into it): one per wave column of every N tile of the SwiGLU-backward GEMM,
// the most any of its kernels uses (256-wide tiles of 64-wide waves; float32
// layers 64-wide tiles of one slot).
inline int dw_slots_max(const ExpertDims& d) {
  return d.dtype == MOE_F32 ? ceil_div(d.I, 64) : ceil_div(d.I, 256) * 4;
}

// Backward workspace: tile lists, G B_d and dH B_gu [N, r], dH [N, 2I],
// split-K and side-product partials; for the combine backward folded in,
// also the permuted routing weights [N] f32, w u_d and w G B_d [N, r] and
// the dw partials [slots, N] f32.
struct BwdWs {
  WsLayout L;
  void *gb, *dhb, *dh, *split;
  float* vpart;
  float* w_perm;
  void *wu_d, *gbw;
  float* dwp;
  size_t bytes;
};

BwdWs bwd_ws(void* ws, const ExpertDims& d) {
  const size_t esz = d.dtype == MOE_F32 ? 4 : 2;
  BwdWs B;
  B.L = tile_ws(ws, d);
  char* base = static_cast<char*>(ws);
  size_t off = B.L.bytes;
  auto take = [&](size_t n) {
    void* q = base ? base + off : nullptr;
    off += align_up(n);
    return q;
  };
  B.gb = take(static_cast<size_t>(d.N) * d.r * esz);
  B.dhb = take(static_cast<size_t>(d.N) * d.r * esz);
  B.dh = take(static_cast<size_t>(d.N) * 2 * d.I * esz);
  B.split = take(lora_wgrad_split_bytes(d));
  B.vpart = static_cast<float*>(take(d.dtype != MOE_F32 ? side_part_bytes(d) : 0));
  B.w_perm = static_cast<float*>(take(static_cast<size_t>(d.N) * 4));
  B.wu_d = take(static_cast<size_t>(d.N) * d.r * esz);
  B.gbw = take(static_cast<size_t>(d.N) * d.r * esz);
  B.dwp = static_cast<float*>(take(static_cast<size_t>(dw_slots_max(d)) * d.N * 4));
  B.bytes = off;
  return B;
}

}  // namespace

size_t experts_bwd_ws_bytes(const ExpertDims& d) { return bwd_ws(nullptr, d).bytes; }

namespace {

// h = X W_gu^T + u_gu B_gu^T ; act = SwiGLU(h)   (tile lists already built)
hipError_t launch_gate_up(const ExpertDims& d, const WsLayout& L, const XRows& x,
                          const int32_t* offsets, const moe_weights& w, const void* u_gu,
                          void* h, void* act, hipStream_t s, KernelTimer* tm) {
  const int H = d.H, I = d.I, r = d.r;
  GemmArgs a = base_args(d, offsets, L.big);
  a.a[0] = opnd_x(x, H, 1, esz_of(d));
  a.b[0] = opnd(w.w_gu, static_cast<int64_t>(2) * I * H, H, 1, true);
  a.a[1] = opnd(u_gu, 0, r, 1, r % 8 == 0);
  a.b[1] = opnd(w.b_gu, static_cast<int64_t>(2) * I * r, r, 1, r % 8 == 0);
  a.K[0] = H;
  a.K[1] = r;
  a.N = 2 * I;
  a.out = h;
  a.ld_out = 2 * I;
  a.out2 = act;
  a.ld_out2 = I;
  TimedScope ts(tm, MOE_K_GATE_UP_FWD, s);
  if (d.dtype != MOE_F32) {
    a.ntn = ceil_div(I, 128);
    return launch_big<GROUP_M, EPI_SWIGLU, true, true, true>(gm_grid(d, L.big, a.ntn), a, s,
                                                              L.big.bm);
  }
  a.ntn = ceil_div(I, 64);
  return launch(gemm_f32<GROUP_M, EPI_SWIGLU, true>, gm_grid(d, L.big, a.ntn), a, s);
}

// Recompute mode: h [N, 2I] and act [N, I] live in scratch after `base_bytes`.
inline size_t lean_extra_bytes(const ExpertDims& d) {
  const size_t esz = d.dtype == MOE_F32 ? 4 : 2;
  return align_up(static_cast<size_t>(d.N) * 2 * d.I * esz) +
         align_up(static_cast<size_t>(d.N) * d.I * esz);
}

inline moe_saved lean_saved(const ExpertDims& d, const moe_saved& sv, void* ws, size_t base_bytes) {
  const size_t esz = d.dtype == MOE_F32 ? 4 : 2;
  moe_saved out = sv;
  char* p = static_cast<char*>(ws) + align_up(base_bytes);
  out.h = p;
  out.act = p + align_up(static_cast<size_t>(d.N) * 2 * d.I * esz);
  return out;
}

}  // namespace

hipError_t launch_experts_fwd(const ExpertDims& d, const XRows& x, const int32_t* offsets,
                              const moe_weights& w, const moe_saved& sv, void* ws,
                              hipStream_t s, KernelTimer* tm) {
  const WsLayout L = tile_ws(ws, d);
  const int H = d.H, I = d.I, r = d.r;
  MOE_TRY(build_tiles(L, offsets, d.E, s));
  {  // u_gu = s X A_gu^T
    TimedScope ts(tm, MOE_K_LORA_SIDE, s);
    MOE_TRY(side_product(d, offsets, L, opnd_x(x, H, 1, esz_of(d)), H, w.a_gu,
                         static_cast<int64_t>(r) * H, 1, sv.u_gu, s));
  }
  MOE_TRY(launch_gate_up(d, L, x, offsets, w, sv.u_gu, sv.h, sv.act, s, tm));
  {  // u_d = s act A_d^T
    TimedScope ts(tm, MOE_K_LORA_SIDE, s);
    MOE_TRY(side_product(d, offsets, L, opnd(sv.act, 0, I, 1, true), I, w.a_d,
                         static_cast<int64_t>(r) * I, 1, sv.u_d, s));
  }
  {  // y_exp = act W_d^T + u_d B_d^T
    GemmArgs a = base_args(d, offsets, L.big);
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
    if (d.dtype != MOE_F32) {
      a.ntn = ceil_div(H, 256);
      MOE_TRY((launch_big<GROUP_M, EPI_STORE, false, true, true>( gm_grid(d, L.big, a.ntn),
                     a, s, L.big.bm)));
    } else {
      a.ntn = ceil_div(H, 64);
      MOE_TRY(launch(gemm_f32<GROUP_M, EPI_STORE, false>, gm_grid(d, L.big, a.ntn), a, s));
    }
  }
  return hipSuccess;
}

hipError_t launch_experts_bwd(const ExpertDims& d, const void* g, const XRows& x,
                              const int32_t* offsets, const moe_weights& w,
                              const moe_saved& sv, void* dx_perm, const moe_lora_grads& gr,
                              const moe_base_grads* base, void* ws, hipStream_t s,
                              KernelTimer* tm, const CombineBwd* cb) {
  const BwdWs B = bwd_ws(ws, d);
  const WsLayout& L = B.L;
  const int H = d.H, I = d.I, r = d.r;
  void* gb = B.gb;    // s G B_d (with cb: s dY B_d, unweighted)
  void* dhb = B.dhb;  // s dH B_gu
  void* dh = B.dh;
  void* split = B.split;
  // The side products G B_d and dH B_gu read the same matrices as the
  // gradients dB_d = G^T u_d and dB_gu = dH^T u_gu; where the shapes allow,
  // one kernel reads each matrix once for both.
  const bool fuse_d = side_fusable(d, H, r) && aligned16(w.b_d);
  const bool fuse_gu = side_fusable(d, 2 * I, r) && aligned16(w.b_gu);

  MOE_TRY(build_tiles(L, offsets, d.E, s));
  // With the combine backward folded in, g holds dY's rows unweighted and
  // every consumer of G = w dY applies w itself: dB_d = dY^T (w u_d); the
  // down backward runs on dY and its epilogue scales the product by w (dw
  // comes from the unweighted product); dA_d = (w s dY B_d)^T act; the full
  // fine-tuning dW_d = (w dY)^T act after the rows are scaled in place.
  // With cb->gather_dy (never with base) those rows are not copied: the
  // GEMMs read row sorted_pair[i] / k of dY for permuted row i.
  const bool dyg = cb && cb->gather_dy;
  if (dyg && base) return hipErrorInvalidValue;
  const XRows dyr{cb ? cb->dy : nullptr, cb ? cb->sorted_pair : nullptr, cb ? cb->k : 1,
                  cb ? cb->T : 0};
  const Opnd g_rows = dyg ? opnd_x(dyr, H, 1, esz_of(d)) : opnd(g, 0, H, 1, true);
  const XRows* g_lx = dyg ? &dyr : nullptr;
  const void* ud_eff = sv.u_d;   // right operand of dB_d
  const void* gb_da = gb;        // left operand of dA_d
  if (cb && !dyg) {
    TimedScope ts(tm, MOE_K_DY_GATHER, s);
    const int64_t row_bytes = static_cast<int64_t>(H) * (d.dtype == MOE_F32 ? 4 : 2);
    MOE_TRY(launch_gather(cb->dy, cb->sorted_pair, offsets, d.E, cb->k, d.N, row_bytes,
                          const_cast<void*>(g), s, nullptr));
  }
  if (cb) {  // w of each permuted row, and w u_d
    TimedScope ts(tm, MOE_K_DW_SUM, s);
    MOE_TRY(launch_perm_weights(d.dtype, cb->topk_w, cb->sorted_pair, d.N, sv.u_d, r, B.w_perm,
                                B.wu_d, s));
    ud_eff = B.wu_d;
    gb_da = B.gbw;
  }
  if (fuse_d) {  // dB_d = G^T u_d [H, r] and gb = s G B_d in one pass over G
    TimedScope ts(tm, MOE_K_LORA_WGRAD, s);
    SideOut so;
    so.bm = w.b_d;
    so.out = gb;
    so.part = B.vpart;
    if (cb) {
      so.roww = B.w_perm;
      so.out_w = B.gbw;
    }
    MOE_TRY(weight_grad(d, offsets, g, H, ud_eff, r, gr.db_d, s, split, &so, nullptr, g_lx));
  } else {  // gb = s G B_d      (B_d[e] is [H, r]: K = H rows, r contiguous)
    TimedScope ts(tm, MOE_K_LORA_SIDE, s);
    MOE_TRY(side_product(d, offsets, L, g_rows, H, w.b_d,
                         static_cast<int64_t>(H) * r, 0, gb, s));
    if (cb) MOE_TRY(scale_rows(d.dtype, gb, B.w_perm, d.N, r, B.gbw, s));
  }
  {  // dAct = G W_d + gb A_d ; dH = SwiGLU'(h) dAct
    GemmArgs a = base_args(d, offsets, L.big);
    a.a[0] = g_rows;
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
    a.ntn = d.dtype != MOE_F32 ? ceil_div(I, 256) : ceil_div(I, 64);
    if (cb) {
      a.roww = B.w_perm;
      a.dwp = B.dwp;
      a.dwp_slots = d.dtype != MOE_F32 ? a.ntn * big_waves_n(a, L.big.bm) : a.ntn;
    }
    {
      TimedScope ts(tm, MOE_K_DOWN_BWD, s);
      if (d.dtype != MOE_F32)
        MOE_TRY((launch_big<GROUP_M, EPI_SWIGLU_BWD, false, true, false>(
                       gm_grid(d, L.big, a.ntn), a, s, L.big.bm)));
      else
        MOE_TRY(launch(gemm_f32<GROUP_M, EPI_SWIGLU_BWD, false>, gm_grid(d, L.big, a.ntn), a, s));
    }
    if (cb) {
      TimedScope ts(tm, MOE_K_DW_SUM, s);
      MOE_TRY(launch_dw_sum(B.dwp, a.dwp_slots, cb->inv_pos,
                            static_cast<int64_t>(cb->T) * cb->k, cb->d_topk_w, s));
    }
  }
  {  // dB_d = G^T u_d  [H, r] (unless fused above) ;  dA_d = gb^T act  [r, I]
    TimedScope ts(tm, MOE_K_LORA_WGRAD, s);
    if (!fuse_d)
      MOE_TRY(weight_grad(d, offsets, g, H, ud_eff, r, gr.db_d, s, split, nullptr, nullptr, g_lx));
    MOE_TRY(weight_grad(d, offsets, gb_da, r, sv.act, I, gr.da_d, s, split));
  }
  if (base) {  // full fine-tuning: dW_d = G^T act  [H, I]
    if (cb) {
      TimedScope ts(tm, MOE_K_ROW_SCALE, s);
      MOE_TRY(scale_rows(d.dtype, g, B.w_perm, d.N, H, const_cast<void*>(g), s));
    }
    TimedScope ts(tm, MOE_K_BASE_WGRAD, s);
    MOE_TRY(weight_grad(d, offsets, g, H, sv.act, I, base->dw_d, s, nullptr));
  }
  if (fuse_gu) {  // dB_gu = dH^T u_gu [2I, r] and dhb = s dH B_gu in one pass over dH
    TimedScope ts(tm, MOE_K_LORA_WGRAD, s);
    SideOut so;
    so.bm = w.b_gu;
    so.out = dhb;
    so.part = B.vpart;
    MOE_TRY(weight_grad(d, offsets, dh, 2 * I, sv.u_gu, r, gr.db_gu, s, split, &so));
  } else {  // dhb = s dH B_gu   (B_gu[e] is [2I, r])
    TimedScope ts(tm, MOE_K_LORA_SIDE, s);
    MOE_TRY(side_product(d, offsets, L, opnd(dh, 0, 2 * I, 1, true), 2 * I, w.b_gu,
                         static_cast<int64_t>(2) * I * r, 0, dhb, s));
  }
  {  // dX = dH W_gu + dhb A_gu
    GemmArgs a = base_args(d, offsets, L.big);
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
    if (d.dtype != MOE_F32) {
      a.ntn = ceil_div(H, 256);
      MOE_TRY((launch_big<GROUP_M, EPI_STORE, false, true, false>( gm_grid(d, L.big, a.ntn),
                     a, s, L.big.bm)));
    } else {
      a.ntn = ceil_div(H, 64);
      MOE_TRY(launch(gemm_f32<GROUP_M, EPI_STORE, false>, gm_grid(d, L.big, a.ntn), a, s));
    }
  }
  {  // dB_gu = dH^T u_gu  [2I, r] (unless fused above) ;  dA_gu = dhb^T X  [r, H]
    TimedScope ts(tm, MOE_K_LORA_WGRAD, s);
    if (!fuse_gu) MOE_TRY(weight_grad(d, offsets, dh, 2 * I, sv.u_gu, r, gr.db_gu, s, split));
    MOE_TRY(weight_grad(d, offsets, dhb, r, x.ptr, H, gr.da_gu, s, split, nullptr, &x));
  }
  if (base) {  // full fine-tuning: dW_gu = dH^T X  [2I, H]
    TimedScope ts(tm, MOE_K_BASE_WGRAD, s);
    MOE_TRY(weight_grad(d, offsets, dh, 2 * I, x.ptr, H, base->dw_gu, s, nullptr, nullptr, &x));
  }
  return hipSuccess;
}

size_t experts_fwd_lean_ws_bytes(const ExpertDims& d) {
  return align_up(experts_fwd_ws_bytes(d)) + lean_extra_bytes(d);
}

size_t experts_bwd_lean_ws_bytes(const ExpertDims& d) {
  return align_up(experts_bwd_ws_bytes(d)) + lean_extra_bytes(d);
}

hipError_t launch_experts_fwd_lean(const ExpertDims& d, const XRows& x,
                                   const int32_t* offsets, const moe_weights& w,
                                   const moe_saved& sv, void* ws, hipStream_t s,
                                   KernelTimer* tm) {
  const moe_saved full = lean_saved(d, sv, ws, experts_fwd_ws_bytes(d));
  return launch_experts_fwd(d, x, offsets, w, full, ws, s, tm);
}

hipError_t launch_experts_bwd_recompute(const ExpertDims& d, const void* g, const XRows& x,
                                        const int32_t* offsets, const moe_weights& w,
                                        const moe_saved& sv, void* dx_perm,
                                        const moe_lora_grads& gr, const moe_base_grads* base,
                                        void* ws, hipStream_t s, KernelTimer* tm,
                                        const CombineBwd* cb) {
  const moe_saved full = lean_saved(d, sv, ws, experts_bwd_ws_bytes(d));
  const WsLayout L = tile_ws(ws, d);
  MOE_TRY(build_tiles(L, offsets, d.E, s));
  MOE_TRY(launch_gate_up(d, L, x, offsets, w, sv.u_gu, full.h, full.act, s, tm));
  return launch_experts_bwd(d, g, x, offsets, w, full, dx_perm, gr, base, ws, s, tm, cb);
}

// ----------------------------------------------------------------- router projection
// logits = x W_r^T (float32 out) and its input gradient dx += d_logits W_r, as
// grouped GEMMs over a single group of all T rows (tile list built on the
// device from offsets {0, T}).
namespace {

__global__ void range_offsets_kernel(int32_t* off, int T) {
  if (threadIdx.x == 0) {
    off[0] = 0;
    off[1] = T;
  }
}

template <typename Elem>
__global__ __launch_bounds__(256) void cast_kernel(const float* __restrict__ src,
                                                   Elem* __restrict__ dst, int64_t n) {
  const int64_t i = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
  if (i < n) dst[i] = from_f32<Elem>(src[i]);
}

// dst += src; with vec, each thread takes 16 bytes (both pointers 16-byte aligned).
template <typename Elem>
__global__ __launch_bounds__(256) void accumulate_kernel(const Elem* __restrict__ src,
                                                         Elem* __restrict__ dst, int64_t n,
                                                         bool vec) {
  constexpr int V = 16 / sizeof(Elem);
  const int64_t t = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
  if (vec) {
    const int64_t i = t * V;
    if (i + V <= n) {
      Elem a[V], b[V];
      *reinterpret_cast<uint4*>(a) = *reinterpret_cast<const uint4*>(src + i);
      *reinterpret_cast<uint4*>(b) = *reinterpret_cast<const uint4*>(dst + i);
#pragma unroll
      for (int j = 0; j < V; ++j) b[j] = from_f32<Elem>(to_f32<Elem>(b[j]) + to_f32<Elem>(a[j]));
      *reinterpret_cast<uint4*>(dst + i) = *reinterpret_cast<const uint4*>(b);
    } else {
      for (int64_t j = i; j < n; ++j)
        dst[j] = from_f32<Elem>(to_f32<Elem>(dst[j]) + to_f32<Elem>(src[j]));
    }
  } else if (t < n) {
    dst[t] = from_f32<Elem>(to_f32<Elem>(dst[t]) + to_f32<Elem>(src[t]));
  }
}

struct RouterWs {
  int32_t* offsets;
  WsLayout L;
  bf16_t* dl16;  // d_logits in bf16 (backward, bf16 layers)
  size_t bytes;
};

RouterWs router_ws(void* ws, int T, int E, int dtype) {
  ExpertDims d{};
  d.N = T;
  d.E = 1;
  d.dtype = dtype;
  d.r = 8;  // tile heights as for a LoRA-friendly rank: 128-row small list
  RouterWs R;
  char* p = static_cast<char*>(ws);
  R.offsets = reinterpret_cast<int32_t*>(p);
  size_t off = kAlign;
  R.L = tile_ws(p ? p + off : nullptr, d);
  off += align_up(R.L.bytes);
  R.dl16 = reinterpret_cast<bf16_t*>(p ? p + off : nullptr);
  off += dtype != MOE_F32 ? align_up(static_cast<size_t>(T) * E * 2) : 0;
  R.bytes = off;
  return R;
}

GemmArgs router_args(const RouterWs& R, int dtype) {
  GemmArgs a{};
  a.dtype = dtype;
  a.a[1] = none();
  a.b[1] = none();
  a.E = 1;
  a.offsets = R.offsets;
  a.tiles = R.L.small.tiles;
  a.ntiles = R.L.small.ntiles;
  a.K[1] = 0;
  a.scale = 1.0f;
  return a;
}

}  // namespace

size_t router_ws_bytes(int T, int E, int dtype) { return router_ws(nullptr, T, E, dtype).bytes; }

hipError_t launch_router_fwd(const void* x, const void* w_r, int T, int H, int E, int dtype,
                             float* logits, void* ws, hipStream_t s, KernelTimer* tm) {
  const RouterWs R = router_ws(ws, T, E, dtype);
  TimedScope ts(tm, MOE_K_ROUTER_FWD, s);
  hipLaunchKernelGGL(range_offsets_kernel, dim3(1), dim3(64), 0, s, R.offsets, T);
  MOE_TRY(build_tiles(R.L, R.offsets, 1, s));
  GemmArgs a = router_args(R, dtype);
  a.a[0] = opnd(x, 0, H, 1, true);
  a.b[0] = opnd(w_r, 0, H, 1, true);
  a.K[0] = H;
  a.N = E;
  a.out = logits;
  a.ld_out = E;
  if (dtype != MOE_F32) {
    a.ntn = ceil_div(E, 64);
    return launch(GEMM16(a.dtype, 128, 64, 32, 64, 64, 3, 2, GROUP_M, EPI_STORE_F32, false, true, true, 0),
                  static_cast<int>(tile_cap(T, 1, R.L.small.bm)) * a.ntn, a, s);
  }
  a.ntn = ceil_div(E, 64);
  return launch(gemm_f32<GROUP_M, EPI_STORE, false>,
                static_cast<int>(tile_cap(T, 1, R.L.small.bm)) * a.ntn, a, s);
}

hipError_t launch_router_bwd(const float* d_logits, const void* w_r, int T, int H, int E,
                             int dtype, void* dx, void* ws, hipStream_t s, KernelTimer* tm) {
  const RouterWs R = router_ws(ws, T, E, dtype);
  TimedScope ts(tm, MOE_K_ROUTER_BWD, s);
  hipLaunchKernelGGL(range_offsets_kernel, dim3(1), dim3(64), 0, s, R.offsets, T);
  MOE_TRY(build_tiles(R.L, R.offsets, 1, s));
  GemmArgs a = router_args(R, dtype);
  a.K[0] = E;
  a.N = H;
  a.out = dx;
  a.ld_out = H;
  if (dtype != MOE_F32) {
    const int64_t n = static_cast<int64_t>(T) * E;
    const dim3 grid(static_cast<unsigned>((n + 255) / 256));
    if (dtype == MOE_F16)
      hipLaunchKernelGGL(cast_kernel<f16_t>, grid, dim3(256), 0, s, d_logits,
                         reinterpret_cast<f16_t*>(R.dl16), n);
    else
      hipLaunchKernelGGL(cast_kernel<bf16_t>, grid, dim3(256), 0, s, d_logits, R.dl16, n);
    a.a[0] = opnd(R.dl16, 0, E, 1, true);
    a.b[0] = opnd(w_r, 0, H, 0, true);  // [K = E][N = H]
    a.ntn = ceil_div(H, 256);
    return launch(GEMM16(a.dtype, 128, 256, 64, 128, 32, 3, 2, GROUP_M, EPI_ADD, false, true, false, 0),
                  static_cast<int>(tile_cap(T, 1, R.L.small.bm)) * a.ntn, a, s);
  }
  a.a[0] = opnd(d_logits, 0, E, 1, true);
  a.b[0] = opnd(w_r, 0, H, 0, true);
  a.ntn = ceil_div(H, 64);
  return launch(gemm_f32<GROUP_M, EPI_ADD, false>,
                static_cast<int>(tile_cap(T, 1, R.L.small.bm)) * a.ntn, a, s);
}

// ----------------------------------------------------------------- merged export
// W'[e] = W[e] + s B[e] A[e] for both stacked projections. 16-bit layers use
// merge_kernel below; float32 layers a grouped GEMM whose "tokens" are the
// output rows of each expert's weight (2I for gate_up, H for down; K = r) and
// whose epilogue adds the base weight read from aux.
namespace {

// One stacked projection, 16-bit layers: W [E][R][C], B [E][R][r],
// A [E][r][C]. One block of four waves per 64-row x 256-column tile of an
// expert's W (grid: x = row tile * ntc + column tile, y = expert); wave w
// takes columns 64w .. 64w+63. The pass is bound by streaming W in and W' out,
// so each wave first issues the rank-r operand loads (small, L2-resident),
// then all of its base-weight loads (8 rows x 64 columns per instruction,
// 16 bytes a lane), and only then waits for the operands: the base weight
// arrives while the product runs on MFMA (k = 16 per step, zero past r). The
// product goes through the wave's own LDS tile, 32 rows at a time, so each
// lane ends with 8 consecutive elements of a row: W' = W + s (B A) as one
// float32 sum, rounded once, stored in 16 bytes. VEC: C % 8 == 0 and W, W'
// 16-byte aligned; otherwise every W / W' element is accessed on its own. W'
// may be W itself: each element is read and written by the same lane.
constexpr int kMergeRows = 64, kMergeCols = 256, kMergeLd = 72;

template <bool F16, bool VEC, int KS>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(VEC ? (KS < 4 ? 4 : 2)
                                                                          : (KS < 2 ? 4 : 2))))
void merge_kernel(const bf16_t* W, const bf16_t* __restrict__ Bm,
                  const bf16_t* __restrict__ Am, bf16_t* out, int R, int C, int r, int ntc,
                  float scale, bool avec, bool bvec) {
  // row stride 72 floats: the two half-waves of a fragment store (rows i and
  // i + 4) fall on disjoint banks
  __shared__ float P[4][32][kMergeLd];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int rt = blockIdx.x / ntc, ct = blockIdx.x - rt * ntc;
  const int row0 = rt * kMergeRows;
  const int col0 = ct * kMergeCols + wave * 64;
  if (col0 >= C) return;  // wave-uniform; the kernel has no block barrier
  const int64_t e = blockIdx.y;
  const bf16_t* We = W + e * R * C;
  bf16_t* Oe = out + e * R * C;
  const uint16_t* Be = reinterpret_cast<const uint16_t*>(Bm) + e * R * r;
  const uint16_t* Ae = reinterpret_cast<const uint16_t*>(Am) + e * r * C;
  const int li = lane & 31, lk = (lane >> 5) * 8;

  // Rank-r operands of all k steps (KS of them cover r, zero past r). A-side
  // fragments are B's rows (the product's rows): 16-byte loads when bvec. The
  // B-side fragments need 8 consecutive k of one column of A ([r][C]), so the
  // wave's 64 columns of A are loaded by rows (16 bytes a lane when avec) and
  // written transposed into the wave's LDS tile, At[column][k], from which
  // each fragment is one 16-byte read. The same LDS later holds the product.
  const int ks_n = (r + 15) / 16;
  uint16_t (*At)[kMergeLd] = reinterpret_cast<uint16_t (*)[kMergeLd]>(P[wave]);
  u32x4 ach[2 * KS];
#pragma unroll
  for (int i = 0; i < 2 * KS; ++i) {  // chunk m: k = m / 8, columns 8 (m % 8) .. + 7
    const int m = i * 64 + lane, k = m >> 3, c = col0 + (m & 7) * 8;
    const uint16_t* src = Ae + static_cast<int64_t>(k) * C + c;
    u32x4 v = {0u, 0u, 0u, 0u};
    if (i < 2 * ks_n && k < r && c < C) {
      if (avec) {
        v = *reinterpret_cast<const u32x4*>(src);
      } else {
#pragma unroll
        for (int t = 0; t < 4; ++t) v[t] = src[2 * t] | (static_cast<uint32_t>(src[2 * t + 1]) << 16);
      }
    }
    ach[i] = v;
  }
  u32x4 fa[KS][2], fb[KS][2];
#pragma unroll
  for (int ks = 0; ks < KS; ++ks) {
#pragma unroll
    for (int f = 0; f < 2; ++f) {
      const int n = row0 + 32 * f + li, k0 = ks * 16 + lk;
      const uint16_t* src = Be + static_cast<int64_t>(n) * r + k0;
      u32x4 v = {0u, 0u, 0u, 0u};
      if (ks < ks_n && n < R) {
        if (bvec) {
          if (k0 < r) v = *reinterpret_cast<const u32x4*>(src);
        } else {
#pragma unroll
          for (int t = 0; t < 4; ++t) {
            const uint32_t lo = k0 + 2 * t < r ? src[2 * t] : 0u;
            const uint32_t hi = k0 + 2 * t + 1 < r ? src[2 * t + 1] : 0u;
            v[t] = lo | (hi << 16);
          }
        }
      }
      fa[ks][f] = v;
    }
  }
  __builtin_amdgcn_sched_barrier(0);

  // base weight: load j covers rows 8j .. 8j+7 of the tile, lane -> row
  // 8j + lane/8, columns lc .. lc+7
  const int lr = lane >> 3, lc = col0 + (lane & 7) * 8;
  u32x4 wv[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    const int row = row0 + 8 * j + lr;
    const bf16_t* src = We + static_cast<int64_t>(row) * C + lc;
    if constexpr (VEC) {
      wv[j] = row < R && lc < C ? __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(src))
                                : u32x4{0u, 0u, 0u, 0u};
    } else {
      uint32_t v[4];
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        const uint32_t lo = row < R && lc + 2 * t < C ? src[2 * t] : 0u;
        const uint32_t hi = row < R && lc + 2 * t + 1 < C ? src[2 * t + 1] : 0u;
        v[t] = lo | (hi << 16);
      }
      wv[j] = u32x4{v[0], v[1], v[2], v[3]};
    }
  }
  __builtin_amdgcn_sched_barrier(0);

  // At: every chunk of k steps below ks_n is written (zeros past r)
#pragma unroll
  for (int i = 0; i < 2 * KS; ++i) {
    if (i < 2 * ks_n) {
      const int m = i * 64 + lane, k = m >> 3, cl = (m & 7) * 8;
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        At[cl + 2 * t][k] = static_cast<uint16_t>(ach[i][t] & 0xffffu);
        At[cl + 2 * t + 1][k] = static_cast<uint16_t>(ach[i][t] >> 16);
      }
    }
  }
  wave_lds_sync();
#pragma unroll
  for (int ks = 0; ks < KS; ++ks)
#pragma unroll
    for (int g = 0; g < 2; ++g)
      fb[ks][g] = ks < ks_n ? *reinterpret_cast<const u32x4*>(&At[32 * g + li][ks * 16 + lk])
                            : u32x4{0u, 0u, 0u, 0u};

  float (*Pw)[kMergeLd] = P[wave];
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    f32x16 acc[2];
#pragma unroll
    for (int g = 0; g < 2; ++g)
#pragma unroll
      for (int q = 0; q < 16; ++q) acc[g][q] = 0.0f;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks)
      if (ks < ks_n)
#pragma unroll
        for (int g = 0; g < 2; ++g)
          acc[g] = mfma32<F16>(__builtin_bit_cast(bf16x8, fa[ks][h]),
                               __builtin_bit_cast(bf16x8, fb[ks][g]), acc[g]);
    wave_lds_sync();  // the At reads (h = 0) or the previous half's reads are done
    // acc[g] register q: product row 8(q/4) + 4(lane/32) + q%4 of this
    // half, column 32g + lane%32 of the wave's 64
#pragma unroll
    for (int g = 0; g < 2; ++g)
#pragma unroll
      for (int q = 0; q < 16; ++q)
        Pw[8 * (q >> 2) + 4 * (lane >> 5) + (q & 3)][32 * g + li] = scale * acc[g][q];
    wave_lds_sync();
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int rl = 8 * j + lr, row = row0 + 32 * h + rl;
      const f32x4 p0 = *reinterpret_cast<const f32x4*>(&Pw[rl][(lane & 7) * 8]);
      const f32x4 p1 = *reinterpret_cast<const f32x4*>(&Pw[rl][(lane & 7) * 8 + 4]);
      float v[8];
      unpack8<F16>(wv[4 * h + j], v);
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        v[t] += p0[t];
        v[4 + t] += p1[t];
      }
      if (row >= R) continue;
      bf16_t* dst = Oe + static_cast<int64_t>(row) * C + lc;
      if constexpr (VEC) {
        if (lc < C) store8<F16>(dst, v);
      } else {
#pragma unroll
        for (int t = 0; t < 8; ++t)
          if (lc + t < C) dst[t] = f32_to_h16<F16>(v[t]);
      }
    }
  }
}

__global__ void uniform_offsets_kernel(int32_t* off, int E, int rows) {
  for (int e = threadIdx.x; e <= E; e += blockDim.x) off[e] = e * rows;
}

struct MergeWs {
  int32_t* offsets;
  WsLayout L;
  size_t bytes;
};

MergeWs merge_ws(void* ws, const ExpertDims& d) {
  MergeWs M;
  char* p = static_cast<char*>(ws);
  M.offsets = reinterpret_cast<int32_t*>(p);
  size_t off = align_up(static_cast<size_t>(d.E + 1) * 4);
  M.L = tile_ws(p ? p + off : nullptr, d);
  M.bytes = off + align_up(M.L.bytes);
  return M;
}

// rows of one expert's output, dims of the workspace-sizing view
ExpertDims merge_dims(const ExpertDims& d, int rows) {
  ExpertDims m = d;
  m.N = d.E * rows;
  return m;
}

hipError_t merge_one(const ExpertDims& d, int rows, int cols, const void* w, const void* a,
                     const void* b, void* out, void* ws, hipStream_t s) {
  if (d.dtype != MOE_F32) {
    const int64_t ntc = ceil_div(cols, kMergeCols), nt = ceil_div(rows, kMergeRows) * ntc;
    if (nt > INT32_MAX || d.r > 64) return hipErrorInvalidValue;
    const bool vec = cols % 8 == 0 && aligned16(w) && aligned16(out);
    const bool f16 = d.dtype == MOE_F16;
    auto pick = [&](auto ks) {
      constexpr int KS = decltype(ks)::value;
      return f16 ? (vec ? merge_kernel<true, true, KS> : merge_kernel<true, false, KS>)
                 : (vec ? merge_kernel<false, true, KS> : merge_kernel<false, false, KS>);
    };
    auto kern = d.r <= 16   ? pick(std::integral_constant<int, 1>())
                : d.r <= 32 ? pick(std::integral_constant<int, 2>())
                            : pick(std::integral_constant<int, 4>());
    hipLaunchKernelGGL(kern, dim3(static_cast<unsigned>(nt), d.E), dim3(256), 0, s,
                       static_cast<const bf16_t*>(w), static_cast<const bf16_t*>(b),
                       static_cast<const bf16_t*>(a), static_cast<bf16_t*>(out), rows, cols, d.r,
                       static_cast<int>(ntc), d.scale, aligned16(a),
                       d.r % 8 == 0 && aligned16(b));
    return hipGetLastError();
  }
  const ExpertDims m = merge_dims(d, rows);
  const MergeWs M = merge_ws(ws, m);
  hipLaunchKernelGGL(uniform_offsets_kernel, dim3(1), dim3(256), 0, s, M.offsets, d.E, rows);
  MOE_TRY(build_tiles(M.L, M.offsets, d.E, s));
  GemmArgs g{};
  g.dtype = d.dtype;
  g.a[1] = none();
  g.b[1] = none();
  g.E = d.E;
  g.offsets = M.offsets;
  g.tiles = M.L.small.tiles;
  g.ntiles = M.L.small.ntiles;
  g.a[0] = opnd(b, 0, d.r, 1, d.r % 8 == 0);                               // B rows: [rows, r]
  g.b[0] = opnd(a, static_cast<int64_t>(d.r) * cols, cols, 0, true);      // A[e]: [K = r][N = cols]
  g.K[0] = d.r;
  g.K[1] = 0;
  g.N = cols;
  g.out = out;
  g.ld_out = cols;
  g.aux = w;
  g.ld_aux = cols;
  g.scale = d.scale;
  const int grid_m = static_cast<int>(tile_cap(m.N, d.E, M.L.small.bm));
  g.ntn = ceil_div(cols, 64);
  return launch(gemm_f32<GROUP_M, EPI_ADD, false>, grid_m * g.ntn, g, s);
}

}  // namespace

size_t merge_ws_bytes(const ExpertDims& d) {
  return std::max(merge_ws(nullptr, merge_dims(d, 2 * d.I)).bytes,
                  merge_ws(nullptr, merge_dims(d, d.H)).bytes);
}

hipError_t launch_merge(const ExpertDims& d, const moe_weights& w, void* w_gu_out, void* w_d_out,
                        void* ws, hipStream_t s, KernelTimer* tm) {
  TimedScope ts(tm, MOE_K_MERGE, s);
  if (w_gu_out) MOE_TRY(merge_one(d, 2 * d.I, d.H, w.w_gu, w.a_gu, w.b_gu, w_gu_out, ws, s));
  if (w_d_out) MOE_TRY(merge_one(d, d.H, d.I, w.w_d, w.a_d, w.b_d, w_d_out, ws, s));
  return hipSuccess;
}

hipError_t launch_accumulate(int dtype, int64_t n, const void* src, void* dst, hipStream_t s,
                             KernelTimer* tm) {
  if (n <= 0) return hipSuccess;
  TimedScope ts(tm, MOE_K_ACCUMULATE, s);
  const dim3 grid(static_cast<unsigned>((n + 255) / 256));
  const bool vec = ((reinterpret_cast<uintptr_t>(src) | reinterpret_cast<uintptr_t>(dst)) & 15) == 0;
  auto go = [&](auto tag) {
    using Elem = decltype(tag);
    constexpr int V = 16 / sizeof(Elem);
    const int64_t threads = vec ? (n + V - 1) / V : n;
    hipLaunchKernelGGL(accumulate_kernel<Elem>, dim3(static_cast<unsigned>((threads + 255) / 256)),
                       dim3(256), 0, s, static_cast<const Elem*>(src), static_cast<Elem*>(dst), n,
                       vec);
  };
  if (dtype == MOE_BF16) go(bf16_t{});
  else if (dtype == MOE_F16) go(f16_t{});
  else go(float{});
  return hipGetLastError();
}

}  // namespace moe
