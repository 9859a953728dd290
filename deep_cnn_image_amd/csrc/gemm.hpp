// MFMA GEMM core for every dense contraction on the AlexNet path: implicit-GEMM
// convolution (forward, data gradient, weight gradient) and the FC layers.
//
//   C[m][n] = sum_k A[m][k] * B[n][k]
//
// A and B are never materialised: an operand loader gathers one BK-wide slice
// of the tile straight from the source tensor into a k-contiguous LDS tile.
// Two LDS buffers alternate so the next slice is fetched while the matrix
// cores work on the current one.  The accumulator tile goes through LDS once
// more so that the epilogue writes 16-byte chunks along n.
//
// bf16 sources contiguous along k (plain rows, implicit im2col) are fetched
// with direct-to-LDS buffer loads (buffer_load_dwordx4 ... lds): the data never
// passes through VGPRs, no ds_write is issued, and a padding element is an
// out-of-range buffer offset, which the hardware returns as zero.  Other
// sources (k-outer operands, fp32) go through registers: 16-byte global loads,
// then ds_write into LDS.
//
// bf16 operands use v_mfma_f32_16x16x32_bf16 (fp32 accumulate); fp32 operands
// use v_mfma_f32_16x16x4_f32.  Four waves per workgroup, 64-wide.
#pragma once
#include "common.hpp"
#include "launch.hpp"

#include <type_traits>
#include <utility>

namespace ax {

constexpr int BK = GEMM_BK;
constexpr int NTHREADS = 256;

template <typename T> struct VecOf { static constexpr int V = 16 / sizeof(T); };
// LDS tile layouts [rows][LS] with an XOR swizzle of the 16-byte granule
// index along k.  MFMA fragment reads touch 16 consecutive rows at one
// granule; the layouts keep those reads and the loaders' writes free of bank
// conflicts (64 banks of 4 bytes).
//
// LayoutKC, for loaders that write whole 16-byte granules of a row
// (k-contiguous sources): unpadded rows, so 16 lanes writing two rows cover
// all banks; the granule is XOR-ed with (row >> 1) & 7 (bf16, 8 granules per
// row) or row & 15 (fp32, 16 granules), which spreads the 16 rows of a
// fragment read over all banks.
template <typename T> struct LayoutKC {
  static constexpr int LS = BK;
  template <int R> static constexpr int tile_elems() { return R * LS; }
  static __device__ __forceinline__ int off(int row, int col) {
    constexpr int G = VecOf<T>::V;
    const int s = sizeof(T) == 2 ? ((row >> 1) & 7) : (row & 15);
    return row * LS + (((col / G) ^ s) * G) + (col % G);
  }
  // bf16 MFMA fragment: rows c0 + (lane & 15), k = kk + 8 (lane >> 4) .. + 7
  static __device__ __forceinline__ bf16x8_t frag(const bf16* t, int c0, int kk, int lane) {
    return *reinterpret_cast<const bf16x8_t*>(t + off(c0 + (lane & 15), kk + (lane >> 4) * 8));
  }
};
// LayoutKO, for k-outer loaders whose transposed pair writes put 16 lanes on
// rows 8 apart: rows padded by one granule and the granule XOR-ed with bits
// 4..6 of the row.
template <typename T> struct LayoutKO {
  static constexpr int LS = BK + VecOf<T>::V;
  template <int R> static constexpr int tile_elems() { return R * LS; }
  static __device__ __forceinline__ int off(int row, int col) {
    constexpr int G = VecOf<T>::V;
    return row * LS + (((col / G) ^ ((row >> 4) & 7)) * G) + (col % G);
  }
  static __device__ __forceinline__ bf16x8_t frag(const bf16* t, int c0, int kk, int lane) {
    return *reinterpret_cast<const bf16x8_t*>(t + off(c0 + (lane & 15), kk + (lane >> 4) * 8));
  }
};

// LayoutTR, for bf16 k-outer operands fetched direct-to-LDS: the tile is kept
// as the source stores it, [BK k-rows][128 operand rows] (256-byte k-rows),
// with the 16-byte granule index XOR-ed with swz(k).  Fragments are read with
// ds_read_b64_tr_b16, which transposes within each 16-lane group: lane i of
// the group receives element i % 4 of the 8-byte chunk addressed by lane
// 4 e + i / 4, as its element e.  Lane t addressing k-row k0 + t / 4 at
// operand rows c0 + 4 (t % 4) .. + 3 thus receives operand row c0 + t,
// k = k0 .. k0 + 3; two such reads (k0 and k0 + 4) make an MFMA fragment.
// swz(k) gives the 16 k-rows one read touches (bits 0..1 and 3 of k differ)
// eight distinct even granule offsets, so each half-wave covers all banks.
struct LayoutTR {
  static constexpr int LS = 128;
  template <int R> static constexpr int tile_elems() {
    static_assert(R <= LS, "operand rows per tile");
    return BK * LS;
  }
  static __device__ __forceinline__ int swz(int k) { return ((k & 3) | ((k >> 1) & 4)) << 1; }
  static __device__ __forceinline__ int off(int k, int col) {
    return k * LS + (((col >> 3) ^ swz(k)) << 3) + (col & 7);
  }
  static __device__ __forceinline__ bf16x8_t frag(const bf16* t, int c0, int kk, int lane) {
    const int q = lane & 15;
    const int k = kk + (lane >> 4) * 8 + (q >> 2), col = c0 + 4 * (q & 3);
    typedef short v4s __attribute__((ext_vector_type(4)));
    typedef short v8s __attribute__((ext_vector_type(8)));
    typedef __attribute__((address_space(3))) v4s lds_v4s;
    const v4s lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4s*)(t + off(k, col)));
    const v4s hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4s*)(t + off(k + 4, col)));
    const v8s both = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
    return __builtin_bit_cast(bf16x8_t, both);
  }
};

// ------------------------------------------------------------------ direct-to-LDS
typedef __attribute__((address_space(3))) void lds_void_t;
constexpr uint32_t BUF_OOB = 0x80000000u;   // >= every buffer size used: reads as zero

// Raw buffer descriptor (stride 0, byte-granular range check) over `bytes`.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t buf_rsrc(const void* p, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(p), 0, (int)bytes, 0x00020000);
}

// 16 bytes per lane from byte offset `off` into LDS at lds + 16 * lane.
__device__ __forceinline__ void dma16(__amdgpu_buffer_rsrc_t rs, uint32_t off, bf16* lds) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (lds_void_t*)lds, 16, (int)off, 0, 0, 0);
}

// Wait until at most N vector-memory operations of this wave are in flight
// (loads complete in order, so the older ones have landed).
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
}

// Waits until at most min(ahead, MAXA) slices of OPS loads each are in flight.
template <int OPS, int MAXA>
__device__ __forceinline__ void wait_ahead(int ahead) {
  if constexpr (MAXA > 0) {
    if (ahead >= MAXA) wait_vmcnt<MAXA * OPS>();
    else wait_ahead<OPS, MAXA - 1>(ahead);
  } else {
    wait_vmcnt<0>();
  }
}

// Waits until at most n (0 <= n <= MAX) vector-memory operations of this
// wave are in flight.
template <int MAX>
__device__ __forceinline__ void wait_vmcnt_at_most(int n) {
  if constexpr (MAX > 0) {
    if (n >= MAX) wait_vmcnt<MAX>();
    else wait_vmcnt_at_most<MAX - 1>(n);
  } else {
    wait_vmcnt<0>();
  }
}

// Calls f(integral_constant<int, I>) for I in the sequence, in order.
template <int... I, class F>
__device__ __forceinline__ void unroll_steps(std::integer_sequence<int, I...>, F&& f) {
  (f(std::integral_constant<int, I>{}), ...);
}

// Workgroup barrier without the memory fence of __syncthreads(), which would
// also wait for every direct-to-LDS load still in flight.  Callers order the
// loads themselves with wait_vmcnt.
__device__ __forceinline__ void lds_barrier() {
  asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

// One wave instruction fills 8 rows (1 KB) of a LayoutKC<bf16> tile.  The R/8
// row slots are dealt to the four waves as j = wave + 4 i; a wave short of a
// slot repeats its own previous one (same bytes to the same place), so every
// wave issues NI loads per k-slice and can wait on a fixed count.  Slot j
// keeps the parity of the wave, so the swizzled k granule a lane fetches is
// fixed for the whole k loop.
template <int R>
struct DmaSlots {
  static_assert(R % 8 == 0, "tile rows");
  static constexpr int NSLOT = R / 8, NI = (NSLOT + 3) / 4;
  static __device__ __forceinline__ int slot(int wave, int i) {
    const int j = wave + 4 * i;
    if constexpr (NSLOT % 4 == 0) return j;   // wave < 4: always in range
    return j < NSLOT ? j : j - 4;
  }
  // k granule (of 8) that `lane` fetches for a slot of parity `odd`
  static __device__ __forceinline__ int granule(int lane, int odd) {
    return (lane & 7) ^ ((odd << 2) | ((lane >> 4) & 3));
  }
};

struct GemmGrid {
  int M, N, K;          // per group
  int tiles_m, tiles_n; // tile counts
  int splits;           // split-K factor
  int groups;           // independent GEMMs (convolution groups)
  int kt_per_split;     // k-tiles per split
  int strip_n;          // tile order: 0 = n fastest over whole rows; w > 0 = strips of w n-tiles (see k_gemm)
};

// ------------------------------------------------------------------ loaders
// Interface: setup(r0, g, k_begin) once per tile, then load() fetches the
// current BK-wide k-slice into registers and steps to the next one, and
// store(lds) writes the registers into the LDS tile [rows][BK + pad].  All
// index decomposition happens in setup(); load() only adds and compares.
//
// K-contiguous sources write 16-byte chunks straight into LDS.  K-outer
// sources (rows contiguous, k outer) are transposed on the way: each thread
// holds two consecutive k-rows of one 16-byte row chunk and writes them as
// 32-bit (bf16) or 64-bit (fp32) pairs.

template <typename T> struct PairStore;
template <> struct PairStore<bf16> {
  // rows e of chunk lo/hi (k, k+1) -> d[e*LS] = (lo_e, hi_e)
  template <int LS>
  static __device__ __forceinline__ void run(bf16* d, uint4 lo, uint4 hi) {
    const uint32_t a[4] = {lo.x, lo.y, lo.z, lo.w}, b[4] = {hi.x, hi.y, hi.z, hi.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      *reinterpret_cast<uint32_t*>(d + (2 * i) * LS) = (a[i] & 0xFFFFu) | (b[i] << 16);
      *reinterpret_cast<uint32_t*>(d + (2 * i + 1) * LS) = (a[i] >> 16) | (b[i] & 0xFFFF0000u);
    }
  }
};
template <> struct PairStore<float> {
  template <int LS>
  static __device__ __forceinline__ void run(float* d, uint4 lo, uint4 hi) {
    const uint32_t a[4] = {lo.x, lo.y, lo.z, lo.w}, b[4] = {hi.x, hi.y, hi.z, hi.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) *reinterpret_cast<uint2*>(d + i * LS) = make_uint2(a[i], b[i]);
  }
};

// Rows contiguous along k: element (r, k) at base[r * ld + k].  Needs K % V == 0
// and 16-byte aligned rows.
template <typename T, int R>
struct LdKC {
  using Layout = LayoutKC<T>;
  static constexpr bool DMA = false;
  static constexpr int V = VecOf<T>::V, CPR = BK / V, NCHUNK = R * CPR;
  static constexpr int NCH = (NCHUNK + NTHREADS - 1) / NTHREADS;
  const T* p; int64_t ld; int rows; int K; int64_t gstride;
  const T* base; int r0, k;
  uint4 reg[NCH];
  __device__ void setup(int r0_, int g, int kb) { r0 = r0_; k = kb; base = p + (int64_t)g * gstride; }
  __device__ void load() {
#pragma unroll
    for (int i = 0; i < NCH; ++i) {
      const int c = threadIdx.x + i * NTHREADS;
      uint4 v = make_uint4(0, 0, 0, 0);
      if (c < NCHUNK) {
        const int r = r0 + c / CPR, kk = k + (c % CPR) * V;
        if (r < rows && kk < K) v = *reinterpret_cast<const uint4*>(base + r * ld + kk);
      }
      reg[i] = v;
    }
    k += BK;
  }
  __device__ void store(T* s) {
#pragma unroll
    for (int i = 0; i < NCH; ++i) {
      const int c = threadIdx.x + i * NTHREADS;
      if (c < NCHUNK) *reinterpret_cast<uint4*>(s + Layout::off(c / CPR, (c % CPR) * V)) = reg[i];
    }
  }
};

// Rows contiguous, k outer: element (r, k) at base[k * ld + r].  Needs
// rows % V == 0.
template <typename T, int R>
struct LdKO {
  using Layout = LayoutKO<T>;
  static constexpr bool DMA = false;
  static constexpr int V = VecOf<T>::V, CPK = R / V, NTASK = (BK / 2) * CPK;
  static constexpr int NT = (NTASK + NTHREADS - 1) / NTHREADS;
  static constexpr int LS = Layout::LS;
  const T* p; int64_t ld; int rows; int K; int64_t gstride;
  const T* base; int r0, k;
  uint4 lo[NT], hi[NT];
  __device__ void setup(int r0_, int g, int kb) { r0 = r0_; k = kb; base = p + (int64_t)g * gstride; }
  __device__ void load() {
#pragma unroll
    for (int i = 0; i < NT; ++i) {
      const int c = threadIdx.x + i * NTHREADS;
      uint4 a = make_uint4(0, 0, 0, 0), b = a;
      if (c < NTASK) {
        const int kk = k + 2 * (c / CPK), r = r0 + (c % CPK) * V;
        if (r < rows) {
          const T* q = base + (int64_t)kk * ld + r;
          if (kk < K) a = *reinterpret_cast<const uint4*>(q);
          if (kk + 1 < K) b = *reinterpret_cast<const uint4*>(q + ld);
        }
      }
      lo[i] = a; hi[i] = b;
    }
    k += BK;
  }
  __device__ void store(T* s) {
#pragma unroll
    for (int i = 0; i < NT; ++i) {
      const int c = threadIdx.x + i * NTHREADS;
      if (c < NTASK) PairStore<T>::template run<LS>(s + Layout::off((c % CPK) * V, 2 * (c / CPK)), lo[i], hi[i]);
    }
  }
};

// Implicit im2col of an NHWC tensor for a convolution (forward, or the data
// gradient as a stride-1 convolution of dY with flipped, transposed weights).
// Row m = (n, ho, wo) over [Nimg][Ho][Wo]; k = (kh, kw, ci) with ci fastest,
// ci < Cg, input channel g*Cg + ci of Ctot.  Needs Cg % V == 0.
struct ConvGeom {
  int H, W, Ctot, Cg, KH, KW, stride, pad, Ho, Wo;
};

template <typename T, int R>
struct LdIm2col {
  using Layout = LayoutKC<T>;
  static constexpr bool DMA = false;
  static constexpr int V = VecOf<T>::V, CPR = BK / V, NCHUNK = R * CPR;
  static constexpr int NCH = (NCHUNK + NTHREADS - 1) / NTHREADS;
  const T* p; ConvGeom cg; int M; int K;
  int hb[NCH], wb[NCH];
  const T* rowp[NCH];
  int kc[NCH], kh[NCH], kw[NCH], ci[NCH];
  uint4 reg[NCH];
  __device__ void setup(int r0, int g, int kb) {
#pragma unroll
    for (int i = 0; i < NCH; ++i) {
      const int c = threadIdx.x + i * NTHREADS;
      const int m = r0 + c / CPR;
      hb[i] = -(1 << 28); wb[i] = 0; rowp[i] = p;
      if (c < NCHUNK && m < M) {
        const int hw = cg.Ho * cg.Wo;
        const int n = m / hw, rem = m - n * hw;
        const int ho = rem / cg.Wo, wo = rem - ho * cg.Wo;
        hb[i] = ho * cg.stride - cg.pad;
        wb[i] = wo * cg.stride - cg.pad;
        rowp[i] = p + (int64_t)n * cg.H * cg.W * cg.Ctot + g * cg.Cg;
      }
      const int k = kb + (c % CPR) * V;
      const int tap = k / cg.Cg;
      kc[i] = k; ci[i] = k - tap * cg.Cg; kh[i] = tap / cg.KW; kw[i] = tap - kh[i] * cg.KW;
    }
  }
  __device__ void load() {
#pragma unroll
    for (int i = 0; i < NCH; ++i) {
      const int c = threadIdx.x + i * NTHREADS;
      uint4 v = make_uint4(0, 0, 0, 0);
      const int hi = hb[i] + kh[i], wi = wb[i] + kw[i];
      if (c < NCHUNK && kc[i] < K && (unsigned)hi < (unsigned)cg.H && (unsigned)wi < (unsigned)cg.W)
        v = *reinterpret_cast<const uint4*>(rowp[i] + ((int64_t)hi * cg.W + wi) * cg.Ctot + ci[i]);
      reg[i] = v;
      kc[i] += BK;
      ci[i] += BK;
      while (ci[i] >= cg.Cg) {
        ci[i] -= cg.Cg;
        if (++kw[i] == cg.KW) { kw[i] = 0; ++kh[i]; }
      }
    }
  }
  __device__ void store(T* s) {
#pragma unroll
    for (int i = 0; i < NCH; ++i) {
      const int c = threadIdx.x + i * NTHREADS;
      if (c < NCHUNK) *reinterpret_cast<uint4*>(s + Layout::off(c / CPR, (c % CPR) * V)) = reg[i];
    }
  }
};

// Direct-to-LDS version of LdKC for bf16: rows of a k-contiguous matrix
// (row stride ld elements, group g at g * gstride).  issue(lds) fetches the
// current k-slice into the tile and steps to the next one.
template <int R>
struct DmaKC {
  static constexpr bool DMA = true;
  using Layout = LayoutKC<bf16>;
  using Slots = DmaSlots<R>;
  static constexpr int NI = Slots::NI;
  const bf16* p; int64_t ld; int rows; int K; int64_t gstride;
  __amdgpu_buffer_rsrc_t rs;
  uint32_t off[NI];
  int kc;
  __device__ void setup(int r0, int g, int kb) {
    const bf16* base = p + (int64_t)g * gstride;
    rs = buf_rsrc(base, (uint32_t)(((int64_t)(rows - 1) * ld + K) * 2));
    const int lane = threadIdx.x & 63, wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int gcol = Slots::granule(lane, wave & 1) * 8;
    kc = kb + gcol;
#pragma unroll
    for (int i = 0; i < NI; ++i) {
      const int r = r0 + Slots::slot(wave, i) * 8 + (lane >> 3);
      off[i] = r < rows ? (uint32_t)((r * ld + kc) * 2) : BUF_OOB;
    }
  }
  __device__ __forceinline__ void issue(bf16* s) {
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const bool kok = kc < K;
#pragma unroll
    for (int i = 0; i < NI; ++i) {
      dma16(rs, kok ? off[i] : BUF_OOB, s + Slots::slot(wave, i) * 8 * BK);
      off[i] += BK * 2;
    }
    kc += BK;
  }
};

// Direct-to-LDS version of LdIm2col for bf16 (same row decomposition).  Two
// k orders: tap-major, k = (kh, kw, ci) as LdIm2col; or, with `blocked` (Cg a
// multiple of BK), channel-blocked k = (ci / BK, kh, kw, ci % BK), where each
// k-slice is one tap of one 64-channel block.  The blocked order revisits a
// block's input rows for every tap before moving on, which keeps a channel
// block of the rows a wave of workgroups touches resident in L2 for wide
// inputs; the weights must be laid out in the same order.
template <int R>
struct DmaIm2col {
  static constexpr bool DMA = true;
  using Layout = LayoutKC<bf16>;
  using Slots = DmaSlots<R>;
  static constexpr int NI = Slots::NI;
  const bf16* p; ConvGeom cg; int M; int K; bool blocked = false;
  __amdgpu_buffer_rsrc_t rs;
  int pix[NI];         // element offset of input pixel (ho s - pad, wo s - pad) of the row's image
  uint32_t skip[NI];   // bit t set: tap t (= kh KW + kw) of the row falls outside the input, or t >= KH KW
  int kh, kw, ci, tap; // blocked: kh, kw, tap uniform, ci = block base + this lane's granule
  __device__ void setup(int r0, int g, int kb) {
    const int lane = threadIdx.x & 63, wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int hw = cg.Ho * cg.Wo;
    const int nimg = (M + hw - 1) / hw;
    rs = buf_rsrc(p, (uint32_t)((int64_t)nimg * cg.H * cg.W * cg.Ctot * 2));
#pragma unroll
    for (int i = 0; i < NI; ++i) {
      const int m = r0 + Slots::slot(wave, i) * 8 + (lane >> 3);
      uint32_t valid = 0;
      pix[i] = 0;
      if (m < M) {
        const int n = m / hw, rem = m - n * hw;
        const int ho = rem / cg.Wo, wo = rem - ho * cg.Wo;
        const int hb = ho * cg.stride - cg.pad, wb = wo * cg.stride - cg.pad;
        pix[i] = ((n * cg.H + hb) * cg.W + wb) * cg.Ctot + g * cg.Cg;
        // taps inside the input: kh in [-hb, H - hb), kw in [-wb, W - wb)
        const int c0 = max(0, -wb), c1 = min(cg.KW, cg.W - wb);
        const int q0 = max(0, -hb), q1 = min(cg.KH, cg.H - hb);
        const uint32_t cols = c1 > c0 ? (1u << c1) - (1u << c0) : 0u;
        for (int q = q0; q < q1; ++q) valid |= cols << (q * cg.KW);
      }
      skip[i] = ~valid;
    }
    const int gcol = Slots::granule(lane, wave & 1) * 8;
    if (blocked) {
      const int kt = kb / BK, taps = cg.KH * cg.KW;
      const int blk = kt / taps;
      tap = kt - blk * taps;
      kh = tap / cg.KW; kw = tap - kh * cg.KW; ci = blk * BK + gcol;
    } else {
      const int kc = kb + gcol;
      tap = kc / cg.Cg;
      ci = kc - tap * cg.Cg; kh = tap / cg.KW; kw = tap - kh * cg.KW;
    }
  }
  // A row's load goes out of range (reads zero) when its tap's skip bit is
  // set: bit 31 of the byte offset, above every buffer size used.  The k
  // tail (k >= K, tap >= KH KW) is covered by the same bits.
  __device__ __forceinline__ void issue(bf16* s) {
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int tapoff = (kh * cg.W + kw) * cg.Ctot + ci;
#pragma unroll
    for (int i = 0; i < NI; ++i) {
      const uint32_t o = ((uint32_t)(pix[i] + tapoff) << 1) | (((skip[i] >> tap) & 1u) << 31);
      dma16(rs, o, s + Slots::slot(wave, i) * 8 * BK);
    }
    if (blocked) {   // K = Cg * KH * KW is a multiple of BK: no k tail
      ++tap;
      if (++kw == cg.KW) { kw = 0; if (++kh == cg.KH) { kh = 0; tap = 0; ci += BK; } }
      return;
    }
    ci += BK;
    while (ci >= cg.Cg) {
      ci -= cg.Cg;
      ++tap;
      if (++kw == cg.KW) { kw = 0; ++kh; }
    }
  }
};
// The skip bits above cover taps 0 .. 31: KH KW taps, plus the k tail of
// the tap-major order, whose last slice reaches at most (BK - 1) / Cg taps
// beyond them.
__host__ __device__ constexpr bool im2col_taps_fit(int KH, int KW, int Cg, bool blocked) {
  return KH * KW + (blocked ? 0 : (BK - 1) / Cg) <= 31;
}

// Output pixel p = (n, ho, wo) over [Nimg][Ho][Wo], stepped by BK at a time.
struct PixelIter {
  int p, n, ho, wo;
  __device__ __forceinline__ void set(int pp, int Ho, int Wo) {
    p = pp; const int hw = Ho * Wo; n = pp / hw; const int rem = pp - n * hw; ho = rem / Wo; wo = rem - ho * Wo;
  }
  __device__ __forceinline__ void advance(int Ho, int Wo) {
    p += BK; wo += BK;
    while (wo >= Wo) { wo -= Wo; if (++ho == Ho) { ho = 0; ++n; } }
  }
};

// Lanes of a direct-to-LDS k-outer tile (LayoutTR): the BK/4 slots of 4
// k-rows (1 KB) are dealt to the waves as j = wave + 4 i.  Lane l fills k-row
// 4 j + l / 16 at physical granule l % 16; the swizzle then maps it to the same
// logical granule (8 operand rows) for every slot of its wave.
struct TrSlots {
  static constexpr int NI = BK / 16;
  static __device__ __forceinline__ int krow(int wave, int i, int lane) { return 4 * (wave + 4 * i) + (lane >> 4); }
  static __device__ __forceinline__ int granule(int wave, int lane) {
    return (lane & 15) ^ LayoutTR::swz(krow(wave, 0, lane));
  }
};

// Direct-to-LDS k-outer operand for bf16: element (r, k) at base[k * ld + r]
// (base = p + g * gstride), r < rows, k < K.
template <int R>
struct DmaKO {
  static constexpr bool DMA = true;
  using Layout = LayoutTR;
  static constexpr int NI = TrSlots::NI;
  const bf16* p; int64_t ld; int rows; int K; int64_t gstride;
  __amdgpu_buffer_rsrc_t rs;
  uint32_t off[NI];
  int kr;          // k of this lane's first slot
  bool cok;
  __device__ void setup(int r0, int g, int kb) {
    const int lane = threadIdx.x & 63, wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    // descriptor based at k-row kb: offsets stay within this split's range
    const int64_t span = ((int64_t)(K - 1 - kb) * ld + rows) * 2;
    rs = buf_rsrc(p + (int64_t)g * gstride + (int64_t)kb * ld, (uint32_t)(span < 0x7FFFFFFF ? span : 0x7FFFFFFF));
    const int col = r0 + TrSlots::granule(wave, lane) * 8;
    cok = col < rows;
    const int k0 = TrSlots::krow(wave, 0, lane);
    kr = kb + k0;
#pragma unroll
    for (int i = 0; i < NI; ++i) off[i] = (uint32_t)(((int64_t)(k0 + 16 * i) * ld + col) * 2);
  }
  __device__ __forceinline__ void issue(bf16* s) {
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
#pragma unroll
    for (int i = 0; i < NI; ++i) {
      const bool ok = cok & (kr + 16 * i < K);
      dma16(rs, ok ? off[i] : BUF_OOB, s + 4 * (wave + 4 * i) * LayoutTR::LS);
      off[i] += (uint32_t)(BK * ld * 2);
    }
    kr += BK;
  }
};

// Direct-to-LDS weight-gradient B operand for bf16 (same element definition
// as LdWgradB below): each lane keeps one operand-row granule, i.e. one tap
// and channel run, and steps its k-rows (output pixels) BK at a time.
template <int R>
struct DmaWgradB {
  static constexpr bool DMA = true;
  using Layout = LayoutTR;
  static constexpr int NI = TrSlots::NI;
  const bf16* p; ConvGeom cg; int rows; int P;   // rows = KH*KW*Cg, P = Nimg*Ho*Wo
  __amdgpu_buffer_rsrc_t rs;
  int hoff, woff, coff, dq, dr;
  bool cok;
  int pn[NI], pho[NI], pwo[NI], pp[NI];
  __device__ void setup(int r0, int g, int kb) {
    const int lane = threadIdx.x & 63, wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int hw = cg.Ho * cg.Wo;
    const int nimg = (P + hw - 1) / hw;
    rs = buf_rsrc(p, (uint32_t)((int64_t)nimg * cg.H * cg.W * cg.Ctot * 2));
    const int r = r0 + TrSlots::granule(wave, lane) * 8;
    cok = r < rows;
    const int rr = cok ? r : 0;
    const int tap = rr / cg.Cg, ci = rr - tap * cg.Cg;
    const int kh = tap / cg.KW, kw = tap - kh * cg.KW;
    hoff = kh - cg.pad; woff = kw - cg.pad; coff = g * cg.Cg + ci;
    dq = BK / cg.Wo; dr = BK - dq * cg.Wo;
#pragma unroll
    for (int i = 0; i < NI; ++i) {
      const int q = kb + TrSlots::krow(wave, i, lane);
      pp[i] = q; pn[i] = q / hw;
      const int rem = q - pn[i] * hw;
      pho[i] = rem / cg.Wo; pwo[i] = rem - pho[i] * cg.Wo;
    }
  }
  __device__ __forceinline__ void issue(bf16* s) {
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
#pragma unroll
    for (int i = 0; i < NI; ++i) {
      const int h = pho[i] * cg.stride + hoff, w = pwo[i] * cg.stride + woff;
      const bool ok = cok & (pp[i] < P) & ((unsigned)h < (unsigned)cg.H) & ((unsigned)w < (unsigned)cg.W);
      const uint32_t o = ok ? (uint32_t)(((pn[i] * cg.H + h) * cg.W + w) * cg.Ctot + coff) * 2u : BUF_OOB;
      dma16(rs, o, s + 4 * (wave + 4 * i) * LayoutTR::LS);
      pp[i] += BK; pwo[i] += dr; pho[i] += dq;
      if (pwo[i] >= cg.Wo) { pwo[i] -= cg.Wo; ++pho[i]; }
      while (pho[i] >= cg.Ho) { pho[i] -= cg.Ho; ++pn[i]; }
    }
  }
};

// Weight gradients sum over all (image, output position) pairs in any order.
// With the batch a multiple of BK, the *pixel-major* order k = pos * Nimg + n
// (image fastest) gives every BK-wide k-slice a single output position pos:
// everything but the image offset of a k-row is then uniform per slice or
// fixed per lane, and the per-slice address work is a handful of scalar and
// vector adds.  Both operands of one GEMM must use the same order.
struct PixMajor {
  int nimg, wo_n;          // images (a multiple of BK), output width
  int n0, pos, ho, wo;     // image of k-row 0 and output position of the current slice
  __device__ void set(int kb, int Nimg, int Wo) {
    nimg = Nimg; wo_n = Wo;
    pos = kb / Nimg; n0 = kb - pos * Nimg; ho = pos / Wo; wo = pos - ho * Wo;
  }
  __device__ __forceinline__ void advance() {
    n0 += BK;
    if (n0 == nimg) { n0 = 0; ++pos; if (++wo == wo_n) { wo = 0; ++ho; } }
  }
};

// DmaKO in pixel-major order for dY^T: element (r, k = pos * Nimg + n) =
// base[(n * HoWo + pos) * ld + r], base = p + g * gstride.
template <int R>
struct DmaKOPix {
  static constexpr bool DMA = true;
  using Layout = LayoutTR;
  static constexpr int NI = TrSlots::NI;
  const bf16* p; int64_t ld; int rows; int Nimg; int HoWo, Wo; int64_t gstride;
  __amdgpu_buffer_rsrc_t rs;
  uint32_t off[NI];   // byte offset of (k-row image, column) relative to image n0, position 0
  PixMajor pm;
  __device__ void setup(int r0, int g, int kb) {
    const int lane = threadIdx.x & 63, wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    rs = buf_rsrc(p + (int64_t)g * gstride, (uint32_t)((int64_t)Nimg * HoWo * ld * 2));
    const int col = r0 + TrSlots::granule(wave, lane) * 8;
#pragma unroll
    for (int i = 0; i < NI; ++i)
      off[i] = col < rows ? (uint32_t)(((int64_t)TrSlots::krow(wave, i, lane) * HoWo * ld + col) * 2) : BUF_OOB;
    pm.set(kb, Nimg, Wo);
  }
  __device__ __forceinline__ void issue(bf16* s) {
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const uint32_t u = (uint32_t)(((int64_t)pm.n0 * HoWo + pm.pos) * ld * 2);
#pragma unroll
    for (int i = 0; i < NI; ++i)
      dma16(rs, off[i] == BUF_OOB ? BUF_OOB : off[i] + u, s + 4 * (wave + 4 * i) * LayoutTR::LS);
    pm.advance();
  }
};

// DmaWgradB in pixel-major order: element (r = (kh, kw, ci), k = pos * Nimg + n) =
// X[n][ho*s - pad + kh][wo*s - pad + kw][g*Cg + ci] with pos = (ho, wo).
template <int R>
struct DmaWgradBPix {
  static constexpr bool DMA = true;
  using Layout = LayoutTR;
  static constexpr int NI = TrSlots::NI;
  const bf16* p; ConvGeom cg; int rows; int Nimg;
  __amdgpu_buffer_rsrc_t rs;
  int hoff, woff, coff;
  bool cok;
  uint32_t roff[NI];   // byte offset of the k-row's image relative to image n0
  PixMajor pm;
  __device__ void setup(int r0, int g, int kb) {
    const int lane = threadIdx.x & 63, wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int64_t img = (int64_t)cg.H * cg.W * cg.Ctot;
    rs = buf_rsrc(p, (uint32_t)(Nimg * img * 2));
    const int r = r0 + TrSlots::granule(wave, lane) * 8;
    cok = r < rows;
    const int rr = cok ? r : 0;
    const int tap = rr / cg.Cg, ci = rr - tap * cg.Cg;
    const int kh = tap / cg.KW, kw = tap - kh * cg.KW;
    hoff = kh - cg.pad; woff = kw - cg.pad; coff = g * cg.Cg + ci;
#pragma unroll
    for (int i = 0; i < NI; ++i) roff[i] = (uint32_t)(TrSlots::krow(wave, i, lane) * img * 2);
    pm.set(kb, Nimg, cg.Wo);
  }
  __device__ __forceinline__ void issue(bf16* s) {
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int h = pm.ho * cg.stride + hoff, w = pm.wo * cg.stride + woff;
    const bool ok = cok & ((unsigned)h < (unsigned)cg.H) & ((unsigned)w < (unsigned)cg.W);
    const uint32_t b = (uint32_t)(((pm.n0 * cg.H + h) * cg.W + w) * cg.Ctot + coff) * 2u;
#pragma unroll
    for (int i = 0; i < NI; ++i) dma16(rs, ok ? roff[i] + b : BUF_OOB, s + 4 * (wave + 4 * i) * LayoutTR::LS);
    pm.advance();
  }
};

// Weight-gradient B operand: element (r = (kh, kw, ci), k = output pixel p) =
// X[n(p)][ho*s - pad + kh][wo*s - pad + kw][g*Cg + ci] of an NHWC tensor.
// Needs Cg % V == 0 (a row chunk never straddles two taps).
template <typename T, int R>
struct LdWgradB {
  using Layout = LayoutKO<T>;
  static constexpr bool DMA = false;
  static constexpr int V = VecOf<T>::V, CPK = R / V, NTASK = (BK / 2) * CPK;
  static constexpr int NT = (NTASK + NTHREADS - 1) / NTHREADS;
  static constexpr int LS = Layout::LS;
  const T* p; ConvGeom cg; int rows; int P;   // rows = KH*KW*Cg, P = Nimg*Ho*Wo
  const T* colp[NT]; int hoff[NT], woff[NT]; bool rok[NT];
  PixelIter it[NT];
  uint4 lo[NT], hi[NT];
  __device__ void setup(int r0, int g, int kb) {
#pragma unroll
    for (int i = 0; i < NT; ++i) {
      const int c = threadIdx.x + i * NTHREADS;
      const int r = r0 + (c % CPK) * V;
      rok[i] = c < NTASK && r < rows;
      const int rr = rok[i] ? r : 0;
      const int tap = rr / cg.Cg, ci = rr - tap * cg.Cg;
      const int kh = tap / cg.KW, kw = tap - kh * cg.KW;
      hoff[i] = kh - cg.pad; woff[i] = kw - cg.pad;
      colp[i] = p + g * cg.Cg + ci;
      it[i].set(kb + 2 * (c / CPK), cg.Ho, cg.Wo);
    }
  }
  __device__ __forceinline__ uint4 fetch(int i, const PixelIter& q) const {
    uint4 v = make_uint4(0, 0, 0, 0);
    const int h = q.ho * cg.stride + hoff[i], w = q.wo * cg.stride + woff[i];
    if (rok[i] && q.p < P && (unsigned)h < (unsigned)cg.H && (unsigned)w < (unsigned)cg.W)
      v = *reinterpret_cast<const uint4*>(colp[i] + (((int64_t)q.n * cg.H + h) * cg.W + w) * cg.Ctot);
    return v;
  }
  __device__ void load() {
#pragma unroll
    for (int i = 0; i < NT; ++i) {
      PixelIter q = it[i];
      lo[i] = fetch(i, q);
      ++q.p; if (++q.wo == cg.Wo) { q.wo = 0; if (++q.ho == cg.Ho) { q.ho = 0; ++q.n; } }
      hi[i] = fetch(i, q);
      it[i].advance(cg.Ho, cg.Wo);
    }
  }
  __device__ void store(T* s) {
#pragma unroll
    for (int i = 0; i < NT; ++i) {
      const int c = threadIdx.x + i * NTHREADS;
      if (c < NTASK) PairStore<T>::template run<LS>(s + Layout::off((c % CPK) * V, 2 * (c / CPK)), lo[i], hi[i]);
    }
  }
};

// ------------------------------------------------------------------ epilogues
// Called for 8 consecutive columns n .. n+7 of row m (n % 8 == 0).

// y = relu(acc + bias) stored as T at out[m*ldo + g*N + n].
template <typename T>
struct EpBiasRelu {
  T* out; const T* bias; int64_t ldo; int M, N;
  __device__ void operator()(int m, int n, int g, int, float* v) const {
    if (m >= M || n >= N) return;
    float b[8];
    Pack8<T>::load(bias + g * N + n, b);
#pragma unroll
    for (int i = 0; i < 8; ++i) { const float t = v[i] + b[i]; v[i] = t > 0.f ? t : 0.f; }
    Pack8<T>::store(out + m * ldo + g * N + n, v);
  }
};

// y = acc * [mask > 0] (mask optional) stored as T at out[m*ldo + g*N + n].
template <typename T>
struct EpMask {
  T* out; const T* mask; int64_t ldo; int M, N;
  __device__ void operator()(int m, int n, int g, int, float* v) const {
    if (m >= M || n >= N) return;
    const int64_t o = m * ldo + g * N + n;
    if (mask) {
      float mk[8];
      Pack8<T>::load(mask + o, mk);
#pragma unroll
      for (int i = 0; i < 8; ++i) v[i] = mk[i] > 0.f ? v[i] : 0.f;
    }
    Pack8<T>::store(out + o, v);
  }
};

// fp32 store to out[((g*splits + s) * M + m) * ldo + n]: split-K partials and
// fp32 weight gradients.
struct EpF32 {
  float* out; int64_t ldo; int M, N, splits;
  __device__ void operator()(int m, int n, int g, int s, float* v) const {
    if (m >= M || n >= N) return;
    float* d = out + ((int64_t)(g * splits + s) * M + m) * ldo + n;
    Pack8<float>::store(d, v);
  }
};

// Epilogue functors may declare `static constexpr bool prefetches = true`,
// a `State`, `State prefetch(m, n)` and `apply(m, n, v, state)`.
template <class EP, class = void>
struct EpPrefetch { static constexpr bool value = false; struct State {}; };
template <class EP>
struct EpPrefetch<EP, std::void_t<typename EP::State>> {
  static constexpr bool value = EP::prefetches;
  using State = typename EP::State;
};

// ------------------------------------------------------------------ MFMA steps
template <typename T, int FM, int FN, class LA, class LB> struct Mma;

template <int FM, int FN, class LA, class LB>
struct Mma<bf16, FM, FN, LA, LB> {
  // All fragments of one BK slice, read before the next slice's loads are
  // issued and multiplied while those loads are in flight.
  struct Frags { bf16x8_t a[BK / 32][FM], b[BK / 32][FN]; };
  static __device__ __forceinline__ void read(const bf16* As, int ra, const bf16* Bs, int rb, Frags& f, int lane) {
#pragma unroll
    for (int s = 0; s < BK / 32; ++s) {
#pragma unroll
      for (int i = 0; i < FM; ++i) f.a[s][i] = LA::frag(As, ra + i * 16, s * 32, lane);
#pragma unroll
      for (int j = 0; j < FN; ++j) f.b[s][j] = LB::frag(Bs, rb + j * 16, s * 32, lane);
    }
  }
  // One 32-deep k-step of the slice.
  struct Half { bf16x8_t a[FM], b[FN]; };
  static __device__ __forceinline__ void read_half(const bf16* As, int ra, const bf16* Bs, int rb, int kk,
                                                   Half& h, int lane) {
#pragma unroll
    for (int i = 0; i < FM; ++i) h.a[i] = LA::frag(As, ra + i * 16, kk, lane);
#pragma unroll
    for (int j = 0; j < FN; ++j) h.b[j] = LB::frag(Bs, rb + j * 16, kk, lane);
  }
  static __device__ __forceinline__ void mul_half(const Half& h, f32x4_t (&acc)[FM][FN]) {
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
      for (int j = 0; j < FN; ++j)
        acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(h.a[i], h.b[j], acc[i][j], 0, 0, 0);
  }
  static __device__ __forceinline__ void mul(const Frags& f, f32x4_t (&acc)[FM][FN]) {
#pragma unroll
    for (int s = 0; s < BK / 32; ++s)
#pragma unroll
      for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int j = 0; j < FN; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(f.a[s][i], f.b[s][j], acc[i][j], 0, 0, 0);
  }
  // As/Bs: LDS tiles; ra/rb: first row of this wave's slice in each tile
  static __device__ __forceinline__ void run(const bf16* As, int ra, const bf16* Bs, int rb,
                                             f32x4_t (&acc)[FM][FN], int lane) {
#pragma unroll
    for (int kk = 0; kk < BK; kk += 32) {
      bf16x8_t a[FM], b[FN];
#pragma unroll
      for (int i = 0; i < FM; ++i) a[i] = LA::frag(As, ra + i * 16, kk, lane);
#pragma unroll
      for (int j = 0; j < FN; ++j) b[j] = LB::frag(Bs, rb + j * 16, kk, lane);
#pragma unroll
      for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int j = 0; j < FN; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[i], b[j], acc[i][j], 0, 0, 0);
    }
  }
};

template <int FM, int FN, class LA, class LB>
struct Mma<float, FM, FN, LA, LB> {
  static __device__ __forceinline__ void run(const float* As, int ra, const float* Bs, int rb,
                                             f32x4_t (&acc)[FM][FN], int lane) {
    const int r = lane & 15, kq = lane >> 4;
#pragma unroll
    for (int kk = 0; kk < BK; kk += 4) {
      float a[FM], b[FN];
#pragma unroll
      for (int i = 0; i < FM; ++i) a[i] = As[LA::off(ra + i * 16 + r, kk + kq)];
#pragma unroll
      for (int j = 0; j < FN; ++j) b[j] = Bs[LB::off(rb + j * 16 + r, kk + kq)];
#pragma unroll
      for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int j = 0; j < FN; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x4f32(a[i], b[j], acc[i][j], 0, 0, 0);
    }
  }
};

// ------------------------------------------------------------------ kernel
// bf16 tiles (up to 192 x 128) run two workgroups per CU, two waves per SIMD;
// one workgroup per CU with larger tiles measured slower (less latency
// hiding).  fp32 tiles run one workgroup per CU.
template <typename T, int BM, int BN>
constexpr int gemm_waves_per_simd() { return sizeof(T) == 2 ? 2 : 1; }
template <typename T, int BM, int BN>
constexpr int gemm_default_stages() { return 2; }
// LDS stages of each operand for the read-ahead schedule of bf16 tiles: the
// A operand (the one gathered from activations: implicit im2col) three, the
// B operand two, for 96-row tiles (3 A + 2 B slices stay within the 80 KB
// that leaves room for a second workgroup on the CU); otherwise two each.
// A slice of A is then requested two slices before it is multiplied instead
// of one.  Measured: 96 x 128 tiles 10% faster; 128 x 128 tiles, whose 3 + 2
// slices take the whole 80 KB, 3-6% slower.
template <typename T, int BM, int BN>
constexpr int gemm_a_stages() {
  return sizeof(T) == 2 && BM <= 96 && (3 * BM + 2 * BN) * GEMM_BK * 2 <= 80 * 1024 ? 3 : 2;
}
// Read-ahead schedule (see k_gemm) for k-contiguous LDS tiles with wave tiles
// of up to 18 fragments, where it measured faster; the slice-at-a-time
// schedule elsewhere (it measured faster with transposing fragment reads and
// with 96 x 64 wave tiles).
template <class LA, class LB, int FM, int FN>
constexpr bool gemm_read_ahead() {
  return std::is_same<LA, LayoutKC<bf16>>::value && std::is_same<LB, LayoutKC<bf16>>::value && FM * FN <= 18;
}

template <typename T, int BM, int BN, int WGM, int WGN, class AL, class BL, class EP, int ST = 2, int STB = ST>
__global__ void __launch_bounds__(NTHREADS)
__attribute__((amdgpu_waves_per_eu(gemm_waves_per_simd<T, BM, BN>(), gemm_waves_per_simd<T, BM, BN>())))
k_gemm(AL al, BL bl, EP ep, GemmGrid gg) {
  static_assert(WGM * WGN == 4, "four waves");
  using LA = typename AL::Layout;
  using LB = typename BL::Layout;
  constexpr int WTM = BM / WGM, WTN = BN / WGN;
  static_assert(WTM % 16 == 0 && WTN % 16 == 0, "wave tile");
  constexpr int FM = WTM / 16, FN = WTN / 16;
  constexpr int A_EL = LA::template tile_elems<BM>(), B_EL = LB::template tile_elems<BN>();
  static_assert(ST >= 2 && (ST == 2 || AL::DMA), "LDS stages: 2, or more with direct-to-LDS operands");
  static_assert(STB == ST || (STB == 2 && ST == 3), "B stages: as many as A, or two beside three");
  constexpr int MAIN_BYTES = (ST * A_EL + STB * B_EL) * (int)sizeof(T);
  constexpr int CST = BN + 4;
  constexpr int EPI_BYTES = WTM * CST * 4;   // one wave row of the tile at a time
  constexpr int SMEM = MAIN_BYTES > EPI_BYTES ? MAIN_BYTES : EPI_BYTES;
  __shared__ __attribute__((aligned(16))) char smem[SMEM];
  T* As = reinterpret_cast<T*>(smem);
  T* Bs = As + ST * A_EL;   // ST A slices, then STB B slices

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);   // uniform: keeps wave offsets scalar
  const int wm = wave / WGN, wn = wave % WGN;

  // Work order.  The 1-D grid enumerates (group, split, tile) with tiles
  // fastest (within a GEMM, n fastest, over whole rows or strips: strip_n).  Hardware deals workgroups round-robin over the eight XCDs, each
  // with its own L2; the remap gives XCD x one contiguous run of that order
  // (the first nb % 8 XCDs one workgroup more), so workgroups that share
  // operand rows (neighbouring tiles, tiles of one split) share an L2.
  const int nb = gridDim.x;
  const int x = blockIdx.x & 7, q = nb >> 3, r = nb & 7;
  const int b = x * q + (x < r ? x : r) + (blockIdx.x >> 3);
  const int tiles = gg.tiles_m * gg.tiles_n;
  const int gs = b / tiles, t = b - gs * tiles;
  const int g = gs / gg.splits, s = gs - g * gg.splits;
  int bm, bn;
  if (gg.strip_n > 0 && gg.strip_n < gg.tiles_n) {
    // column strips of strip_n n-tiles, n fastest within a strip, strips one
    // after the other: the workgroups an XCD runs at once share one strip's
    // B blocks over several rows of tiles, so those stay in L2 while the
    // rows go by
    const int per = gg.strip_n * gg.tiles_m, sidx = t / per, n0s = sidx * gg.strip_n;
    const int wdt = min(gg.tiles_n - n0s, gg.strip_n), r = t - sidx * per;
    bm = r / wdt;
    bn = n0s + (r - bm * wdt);
  } else {
    bm = t / gg.tiles_n;
    bn = t - bm * gg.tiles_n;
  }
  const int m0 = bm * BM, n0 = bn * BN;
  const int total_kt = (gg.K + BK - 1) / BK;
  const int kt0 = s * gg.kt_per_split;
  const int kt1 = min(kt0 + gg.kt_per_split, total_kt);

  al.setup(m0, g, kt0 * BK);
  bl.setup(n0, g, kt0 * BK);
  f32x4_t acc[FM][FN];
#pragma unroll
  for (int i = 0; i < FM; ++i)
#pragma unroll
    for (int j = 0; j < FN; ++j) acc[i][j] = f32x4_t{0.f, 0.f, 0.f, 0.f};

  static_assert(AL::DMA == BL::DMA, "both operands direct-to-LDS or neither");
  if constexpr (AL::DMA) {
    // ST LDS buffers, slice kt in buffer (kt - kt0) % ST.  Both schedules
    // unroll the loop by ST so that buffer offsets are compile-time constants.
    using MM = Mma<T, FM, FN, LA, LB>;
    constexpr int OPS = AL::NI + BL::NI;   // loads per wave per slice
    constexpr bool RA = gemm_read_ahead<LA, LB, FM, FN>();
    static_assert(STB == ST || RA, "fewer B stages only with the read-ahead schedule");
    if constexpr (RA && STB != ST) {
      // Read-ahead with three A stages and two B stages.  At the middle of
      // slice kt, once every wave is done with that slice, B(kt + 2) and then
      // A(kt + 3) are issued into its buffers.  Loads complete in order, so
      // waiting for B(kt + 1) (issued one slice earlier, followed only by
      // A(kt + 2)) also waits for A(kt + 1) and leaves A(kt + 2) in flight.
      // The prologue issues the same sequence: A(0); B(0), A(1); B(1), A(2).
      if (kt0 < kt1) {
        constexpr int NA = AL::NI, NB = BL::NI;
        static_assert(2 * NA + NB < 64, "vmcnt range");
        const int ra = wm * WTM, rb = wn * WTN;
        al.issue(As);
        int after_b0 = 0;   // loads issued after B(kt0)
        bl.issue(Bs);
        if (kt0 + 1 < kt1) { al.issue(As + A_EL); after_b0 += NA; }
        if (kt0 + 1 < kt1) { bl.issue(Bs + B_EL); after_b0 += NB; }
        if (kt0 + 2 < kt1) { al.issue(As + 2 * A_EL); after_b0 += NA; }
        wait_vmcnt_at_most<2 * NA + NB>(after_b0);
        lds_barrier();
        typename MM::Half h0, h1;
        MM::read_half(As, ra, Bs, rb, 0, h0, lane);
        auto step = [&](auto cur_c, int kt) __attribute__((always_inline)) {
          constexpr int CA = decltype(cur_c)::value % 3, CB = decltype(cur_c)::value % 2;
          constexpr int NXA = (CA + 1) % 3, NXB = (CB + 1) % 2;
          MM::read_half(As + CA * A_EL, ra, Bs + CB * B_EL, rb, 32, h1, lane);
          MM::mul_half(h0, acc);
          __builtin_amdgcn_sched_barrier(0);
          const bool more = kt + 1 < kt1;
          if (more) {
            if (kt + 2 < kt1) wait_vmcnt<NA>();   // A(kt + 2) may stay in flight
            else wait_vmcnt<0>();
          }
          lds_barrier();
          if (kt + 2 < kt1) bl.issue(Bs + CB * B_EL);
          if (kt + 3 < kt1) al.issue(As + CA * A_EL);
          __builtin_amdgcn_sched_barrier(0);
          if (more) MM::read_half(As + NXA * A_EL, ra, Bs + NXB * B_EL, rb, 0, h0, lane);
          MM::mul_half(h1, acc);
          __builtin_amdgcn_sched_barrier(0);
        };
        int kt = kt0;
        for (; kt + 5 < kt1; kt += 6)
          unroll_steps(std::make_integer_sequence<int, 6>{},
                       [&](auto i) __attribute__((always_inline)) { step(i, kt + decltype(i)::value); });
        unroll_steps(std::make_integer_sequence<int, 5>{}, [&](auto i) __attribute__((always_inline)) {
          if (kt + decltype(i)::value < kt1) step(i, kt + decltype(i)::value);
        });
      }
    } else if constexpr (RA) {
      // Read-ahead: slice kt sits in buffer (kt - kt0) % ST and up to ST
      // slices are in flight.  Each k-step's fragments are read while the
      // matrix cores multiply the previous k-step's, so no product waits on
      // an LDS read issued just before it.  Between the two k-steps of a
      // slice a wave waits for its own loads of the next slice, and the
      // barrier publishes that slice from every wave; it also marks this
      // slice's buffer as read by all waves, so the loads of slice kt + ST
      // are issued into it right away.
      if (kt0 < kt1) {
        static_assert((ST - 1) * OPS < 64, "vmcnt range");
        const int ra = wm * WTM, rb = wn * WTN;
#pragma unroll
        for (int p = 0; p < ST; ++p)
          if (kt0 + p < kt1) { al.issue(As + p * A_EL); bl.issue(Bs + p * B_EL); }
        wait_ahead<OPS, ST - 1>(kt1 - 1 - kt0);
        lds_barrier();
        typename MM::Half h0, h1;
        MM::read_half(As, ra, Bs, rb, 0, h0, lane);
        auto step = [&](auto cur_c, int kt) __attribute__((always_inline)) {
          constexpr int CUR = decltype(cur_c)::value;
          constexpr int NXT = (CUR + 1) % ST;
          MM::read_half(As + CUR * A_EL, ra, Bs + CUR * B_EL, rb, 32, h1, lane);
          MM::mul_half(h0, acc);
          __builtin_amdgcn_sched_barrier(0);
          const bool more = kt + 1 < kt1;
          if (more) wait_ahead<OPS, ST - 2>(kt1 - 2 - kt);
          lds_barrier();
          if (kt + ST < kt1) { al.issue(As + CUR * A_EL); bl.issue(Bs + CUR * B_EL); }
          __builtin_amdgcn_sched_barrier(0);
          if (more) MM::read_half(As + NXT * A_EL, ra, Bs + NXT * B_EL, rb, 0, h0, lane);
          MM::mul_half(h1, acc);
          __builtin_amdgcn_sched_barrier(0);
        };
        int kt = kt0;
        for (; kt + ST - 1 < kt1; kt += ST)
          unroll_steps(std::make_integer_sequence<int, ST>{},
                       [&](auto i) __attribute__((always_inline)) { step(i, kt + decltype(i)::value); });
        unroll_steps(std::make_integer_sequence<int, ST - 1>{}, [&](auto i) __attribute__((always_inline)) {
          if (kt + decltype(i)::value < kt1) step(i, kt + decltype(i)::value);
        });
      }
    } else if (kt0 < kt1) {
      // Slice-at-a-time: up to ST - 1 slices in flight.  At the top of an
      // iteration a wave waits until its own loads of slice kt have landed
      // (loads complete in order, so it may leave the later slices
      // outstanding); the barrier then publishes the slice from every wave and
      // guarantees that all waves are done with the buffer read one iteration
      // earlier, which the slice ST - 1 ahead then overwrites while the matrix
      // cores work.  All fragments of the slice are read into registers before
      // those loads are issued, so no LDS read has to wait for them.
      static_assert((ST - 2) * OPS < 64, "vmcnt range");
#pragma unroll
      for (int p = 0; p < ST - 1; ++p)
        if (kt0 + p < kt1) { al.issue(As + p * A_EL); bl.issue(Bs + p * B_EL); }
      auto step = [&](auto cur_c, int kt) __attribute__((always_inline)) {
        constexpr int CUR = decltype(cur_c)::value;
        const int ahead = kt1 - 1 - kt;   // slices issued after this one: min(ahead, ST - 2)
        wait_ahead<OPS, ST - 2>(ahead);
        lds_barrier();
        typename MM::Frags f;
        MM::read(As + CUR * A_EL, wm * WTM, Bs + CUR * B_EL, wn * WTN, f, lane);
        __builtin_amdgcn_sched_barrier(0);
        if (kt + ST - 1 < kt1) {
          constexpr int NXT = (CUR + ST - 1) % ST;
          al.issue(As + NXT * A_EL);
          bl.issue(Bs + NXT * B_EL);
        }
        __builtin_amdgcn_sched_barrier(0);
        MM::mul(f, acc);
        // keep the next slice's wait and barrier behind these products
        __builtin_amdgcn_sched_barrier(0);
      };
      int kt = kt0;
      for (; kt + ST - 1 < kt1; kt += ST)
        unroll_steps(std::make_integer_sequence<int, ST>{},
                     [&](auto i) __attribute__((always_inline)) { step(i, kt + decltype(i)::value); });
      unroll_steps(std::make_integer_sequence<int, ST - 1>{}, [&](auto i) __attribute__((always_inline)) {
        if (kt + decltype(i)::value < kt1) step(i, kt + decltype(i)::value);
      });
    }
    lds_barrier();   // all fragment reads done before the epilogue reuses LDS
  } else if (kt0 < kt1) {
    al.load();
    bl.load();
    al.store(As);
    bl.store(Bs);
    __syncthreads();
    for (int kt = kt0; kt < kt1; ++kt) {
      const int cur = (kt - kt0) & 1;
      const bool more = kt + 1 < kt1;
      if (more) { al.load(); bl.load(); }
      Mma<T, FM, FN, LA, LB>::run(As + cur * A_EL, wm * WTM, Bs + cur * B_EL, wn * WTN, acc, lane);
      if (more) { al.store(As + (cur ^ 1) * A_EL); bl.store(Bs + (cur ^ 1) * B_EL); }
      __syncthreads();
    }
  }

  // Epilogue, one wave row (WTM rows of the tile) at a time: the waves of
  // that row stage their accumulators in LDS as fp32, then all threads hand
  // 8-column runs to the epilogue functor.
  float* Cs = reinterpret_cast<float*>(smem);
  constexpr int CPRO = BN / 8, NOUT = WTM * CPRO;
  // Functors that read memory per output chunk (EpPrefetch) issue those
  // reads for all of this thread's chunks before the staging, so they are in
  // flight while the accumulators go through LDS.
  constexpr bool PRE = EpPrefetch<EP>::value && NOUT % NTHREADS == 0;
  constexpr int CH = PRE ? NOUT / NTHREADS : 1;
#pragma unroll 1
  for (int pr = 0; pr < WGM; ++pr) {
    typename EpPrefetch<EP>::State pre[CH];
    if constexpr (PRE) {
#pragma unroll
      for (int i = 0; i < CH; ++i) {
        const int c = tid + i * NTHREADS, r = c / CPRO, cn = (c - r * CPRO) * 8;
        pre[i] = ep.prefetch(m0 + pr * WTM + r, n0 + cn);
      }
    }
    if (pr > 0) __syncthreads();
    if (wm == pr) {
      const int cr = (lane >> 4) * 4, cc = lane & 15;
#pragma unroll
      for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int j = 0; j < FN; ++j)
#pragma unroll
          for (int q = 0; q < 4; ++q)
            Cs[(i * 16 + cr + q) * CST + wn * WTN + j * 16 + cc] = acc[i][j][q];
    }
    __syncthreads();
    if constexpr (PRE) {
#pragma unroll
      for (int i = 0; i < CH; ++i) {
        const int c = tid + i * NTHREADS, r = c / CPRO, cn = (c - r * CPRO) * 8;
        float v[8];
        const float* src = Cs + r * CST + cn;
#pragma unroll
        for (int q = 0; q < 8; ++q) v[q] = src[q];
        ep.apply(m0 + pr * WTM + r, n0 + cn, v, pre[i]);
      }
    } else {
      for (int c = tid; c < NOUT; c += NTHREADS) {
        const int r = c / CPRO, cn = (c - r * CPRO) * 8;
        float v[8];
        const float* src = Cs + r * CST + cn;
#pragma unroll
        for (int i = 0; i < 8; ++i) v[i] = src[i];
        ep(m0 + pr * WTM + r, n0 + cn, g, s, v);
      }
    }
  }
}

}  // namespace ax
