// MFMA GEMM core for every dense contraction on the AlexNet path: implicit-GEMM
// convolution (forward, data gradient, weight gradient) and the FC layers.
//
//   C[m][n] = sum_k A[m][k] * B[n][k]
//
// A and B are never materialised: an operand loader gathers one BK-wide slice
// of the tile straight from the source tensor into registers (16-byte vector
// loads where the source is contiguous along k or along rows) and writes it to
// LDS in a k-contiguous layout [rows][BK + pad].  Two LDS buffers alternate so
// the next slice is fetched while the matrix cores work on the current one.
// The accumulator tile goes through LDS once more so that the epilogue writes
// 16-byte chunks along n.
//
// bf16 operands use v_mfma_f32_16x16x32_bf16 (fp32 accumulate); fp32 operands
// use v_mfma_f32_16x16x4_f32.  Four waves per workgroup, 64-wide.
#pragma once
#include "common.hpp"
#include "launch.hpp"

namespace ax {

constexpr int BK = GEMM_BK;
constexpr int NTHREADS = 256;

template <typename T> struct VecOf { static constexpr int V = 16 / sizeof(T); };
template <typename T> struct Lds { static constexpr int LS = BK + VecOf<T>::V; };  // padded row

// LDS element offset of (row, col) in a [rows][LS] tile.  The 16-byte granule
// index along k is XOR-ed with bits 4..6 of the row: the transposed pair
// writes of k-outer loaders (16 lanes on rows 8 apart) then spread over all
// banks, while the MFMA fragment reads (16 consecutive rows, same granule)
// see one constant permutation and stay conflict-free thanks to the pad.
template <typename T>
__device__ __forceinline__ int lds_off(int row, int col) {
  constexpr int G = VecOf<T>::V;
  return row * Lds<T>::LS + (((col / G) ^ ((row >> 4) & 7)) * G) + (col % G);
}

struct GemmGrid {
  int M, N, K;          // per group
  int tiles_m, tiles_n; // tile counts
  int splits;           // split-K factor (blockIdx.z = group * splits + split)
  int kt_per_split;     // k-tiles per split
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
  static constexpr int V = VecOf<T>::V, CPR = BK / V, NCHUNK = R * CPR;
  static constexpr int NCH = (NCHUNK + NTHREADS - 1) / NTHREADS;
  static constexpr int LS = Lds<T>::LS;
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
      if (c < NCHUNK) *reinterpret_cast<uint4*>(s + lds_off<T>(c / CPR, (c % CPR) * V)) = reg[i];
    }
  }
};

// Rows contiguous, k outer: element (r, k) at base[k * ld + r].  Needs
// rows % V == 0.
template <typename T, int R>
struct LdKO {
  static constexpr int V = VecOf<T>::V, CPK = R / V, NTASK = (BK / 2) * CPK;
  static constexpr int NT = (NTASK + NTHREADS - 1) / NTHREADS;
  static constexpr int LS = Lds<T>::LS;
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
      if (c < NTASK) PairStore<T>::template run<LS>(s + lds_off<T>((c % CPK) * V, 2 * (c / CPK)), lo[i], hi[i]);
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
  static constexpr int V = VecOf<T>::V, CPR = BK / V, NCHUNK = R * CPR;
  static constexpr int NCH = (NCHUNK + NTHREADS - 1) / NTHREADS;
  static constexpr int LS = Lds<T>::LS;
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
      if (c < NCHUNK) *reinterpret_cast<uint4*>(s + lds_off<T>(c / CPR, (c % CPR) * V)) = reg[i];
    }
  }
};

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

// Weight-gradient B operand: element (r = (kh, kw, ci), k = output pixel p) =
// X[n(p)][ho*s - pad + kh][wo*s - pad + kw][g*Cg + ci] of an NHWC tensor.
// Needs Cg % V == 0 (a row chunk never straddles two taps).
template <typename T, int R>
struct LdWgradB {
  static constexpr int V = VecOf<T>::V, CPK = R / V, NTASK = (BK / 2) * CPK;
  static constexpr int NT = (NTASK + NTHREADS - 1) / NTHREADS;
  static constexpr int LS = Lds<T>::LS;
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
      if (c < NTASK) PairStore<T>::template run<LS>(s + lds_off<T>((c % CPK) * V, 2 * (c / CPK)), lo[i], hi[i]);
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

// ------------------------------------------------------------------ MFMA steps
template <typename T, int FM, int FN> struct Mma;

template <int FM, int FN>
struct Mma<bf16, FM, FN> {
  // As/Bs: LDS tiles; ra/rb: first row of this wave's slice in each tile
  static __device__ __forceinline__ void run(const bf16* As, int ra, const bf16* Bs, int rb,
                                             f32x4_t (&acc)[FM][FN], int lane) {
    const int r = lane & 15, kq = (lane >> 4) * 8;
#pragma unroll
    for (int kk = 0; kk < BK; kk += 32) {
      bf16x8_t a[FM], b[FN];
#pragma unroll
      for (int i = 0; i < FM; ++i)
        a[i] = *reinterpret_cast<const bf16x8_t*>(As + lds_off<bf16>(ra + i * 16 + r, kk + kq));
#pragma unroll
      for (int j = 0; j < FN; ++j)
        b[j] = *reinterpret_cast<const bf16x8_t*>(Bs + lds_off<bf16>(rb + j * 16 + r, kk + kq));
#pragma unroll
      for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int j = 0; j < FN; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[i], b[j], acc[i][j], 0, 0, 0);
    }
  }
};

template <int FM, int FN>
struct Mma<float, FM, FN> {
  static __device__ __forceinline__ void run(const float* As, int ra, const float* Bs, int rb,
                                             f32x4_t (&acc)[FM][FN], int lane) {
    const int r = lane & 15, kq = lane >> 4;
#pragma unroll
    for (int kk = 0; kk < BK; kk += 4) {
      float a[FM], b[FN];
#pragma unroll
      for (int i = 0; i < FM; ++i) a[i] = As[lds_off<float>(ra + i * 16 + r, kk + kq)];
#pragma unroll
      for (int j = 0; j < FN; ++j) b[j] = Bs[lds_off<float>(rb + j * 16 + r, kk + kq)];
#pragma unroll
      for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int j = 0; j < FN; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x4f32(a[i], b[j], acc[i][j], 0, 0, 0);
    }
  }
};

// ------------------------------------------------------------------ kernel
template <typename T, int BM, int BN, int WGM, int WGN, class AL, class BL, class EP>
__global__ void __launch_bounds__(NTHREADS) k_gemm(AL al, BL bl, EP ep, GemmGrid gg) {
  static_assert(WGM * WGN == 4, "four waves");
  constexpr int LS = Lds<T>::LS;
  constexpr int WTM = BM / WGM, WTN = BN / WGN;
  static_assert(WTM % 16 == 0 && WTN % 16 == 0, "wave tile");
  constexpr int FM = WTM / 16, FN = WTN / 16;
  constexpr int A_EL = BM * LS, B_EL = BN * LS;
  constexpr int MAIN_BYTES = 2 * (A_EL + B_EL) * (int)sizeof(T);
  constexpr int CST = BN + 4;
  constexpr int EPI_BYTES = BM * CST * 4;
  constexpr int SMEM = MAIN_BYTES > EPI_BYTES ? MAIN_BYTES : EPI_BYTES;
  __shared__ __attribute__((aligned(16))) char smem[SMEM];
  T* As = reinterpret_cast<T*>(smem);
  T* Bs = As + 2 * A_EL;

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave / WGN, wn = wave % WGN;

  // Tile order: consecutive logical tiles (same m-row, neighbouring n) are kept
  // on one XCD so they share its L2; hardware deals workgroups round-robin
  // over the eight XCDs.
  const int nb = gridDim.x;
  int b = blockIdx.x;
  if ((nb & 7) == 0) b = (b & 7) * (nb >> 3) + (b >> 3);
  const int bm = b / gg.tiles_n, bn = b - bm * gg.tiles_n;
  const int g = blockIdx.z / gg.splits, s = blockIdx.z - g * gg.splits;
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

  if (kt0 < kt1) {
    al.load();
    bl.load();
    al.store(As);
    bl.store(Bs);
    __syncthreads();
    for (int kt = kt0; kt < kt1; ++kt) {
      const int cur = (kt - kt0) & 1;
      const bool more = kt + 1 < kt1;
      if (more) { al.load(); bl.load(); }
      Mma<T, FM, FN>::run(As + cur * A_EL, wm * WTM, Bs + cur * B_EL, wn * WTN, acc, lane);
      if (more) { al.store(As + (cur ^ 1) * A_EL); bl.store(Bs + (cur ^ 1) * B_EL); }
      __syncthreads();
    }
  }

  // accumulators -> LDS tile [BM][BN] fp32
  float* Cs = reinterpret_cast<float*>(smem);
  {
    const int cr = (lane >> 4) * 4, cc = lane & 15;
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
      for (int j = 0; j < FN; ++j)
#pragma unroll
        for (int q = 0; q < 4; ++q)
          Cs[(wm * WTM + i * 16 + cr + q) * CST + wn * WTN + j * 16 + cc] = acc[i][j][q];
  }
  __syncthreads();
  constexpr int CPRO = BN / 8, NOUT = BM * CPRO;
  for (int c = tid; c < NOUT; c += NTHREADS) {
    const int r = c / CPRO, cn = (c - r * CPRO) * 8;
    float v[8];
    const float* src = Cs + r * CST + cn;
#pragma unroll
    for (int i = 0; i < 8; ++i) v[i] = src[i];
    ep(m0 + r, n0 + cn, g, s, v);
  }
}

}  // namespace ax
