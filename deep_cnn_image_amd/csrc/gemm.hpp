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

namespace ax {

constexpr int BK = 32;
constexpr int NTHREADS = 256;

template <typename T> struct VecOf { static constexpr int V = 16 / sizeof(T); };
template <typename T> struct Lds { static constexpr int LS = BK + VecOf<T>::V; };  // padded row

struct GemmGrid {
  int M, N, K;          // per group
  int tiles_m, tiles_n; // tile counts
  int splits;           // split-K factor (blockIdx.z = group * splits + split)
  int kt_per_split;     // k-tiles per split
};

// ------------------------------------------------------------------ loaders
// Common shape: chunk c of the tile covers V consecutive elements.

// Rows contiguous along k: element (r, k) at base[r * ld + k].  Needs K % V == 0
// and 16-byte aligned rows.
template <typename T, int R>
struct LdKC {
  static constexpr int V = VecOf<T>::V, CPR = BK / V, NCHUNK = R * CPR;
  static constexpr int NCH = (NCHUNK + NTHREADS - 1) / NTHREADS;
  static constexpr int LS = Lds<T>::LS;
  const T* p; int64_t ld; int rows; int K; int64_t gstride;
  const T* base; int r0;
  uint4 reg[NCH];
  __device__ void setup(int r0_, int g) { r0 = r0_; base = p + (int64_t)g * gstride; }
  __device__ void load(int k0) {
#pragma unroll
    for (int i = 0; i < NCH; ++i) {
      const int c = threadIdx.x + i * NTHREADS;
      uint4 v = make_uint4(0, 0, 0, 0);
      if (c < NCHUNK) {
        const int r = r0 + c / CPR, k = k0 + (c % CPR) * V;
        if (r < rows && k < K) v = *reinterpret_cast<const uint4*>(base + r * ld + k);
      }
      reg[i] = v;
    }
  }
  __device__ void store(T* s) {
#pragma unroll
    for (int i = 0; i < NCH; ++i) {
      const int c = threadIdx.x + i * NTHREADS;
      if (c < NCHUNK) *reinterpret_cast<uint4*>(s + (c / CPR) * LS + (c % CPR) * V) = reg[i];
    }
  }
};

// Rows contiguous, k outer: element (r, k) at base[k * ld + r].  Needs
// rows % V == 0.  The slice is transposed on its way into LDS.
template <typename T, int R>
struct LdKO {
  static constexpr int V = VecOf<T>::V, CPK = R / V, NCHUNK = BK * CPK;
  static constexpr int NCH = (NCHUNK + NTHREADS - 1) / NTHREADS;
  static constexpr int LS = Lds<T>::LS;
  const T* p; int64_t ld; int rows; int K; int64_t gstride;
  const T* base; int r0;
  uint4 reg[NCH];
  __device__ void setup(int r0_, int g) { r0 = r0_; base = p + (int64_t)g * gstride; }
  __device__ void load(int k0) {
#pragma unroll
    for (int i = 0; i < NCH; ++i) {
      const int c = threadIdx.x + i * NTHREADS;
      uint4 v = make_uint4(0, 0, 0, 0);
      if (c < NCHUNK) {
        const int k = k0 + c / CPK, r = r0 + (c % CPK) * V;
        if (r < rows && k < K) v = *reinterpret_cast<const uint4*>(base + (int64_t)k * ld + r);
      }
      reg[i] = v;
    }
  }
  __device__ void store(T* s) {
#pragma unroll
    for (int i = 0; i < NCH; ++i) {
      const int c = threadIdx.x + i * NTHREADS;
      if (c < NCHUNK) {
        T e[V];
        unpack_u4(reg[i], e);
        T* d = s + (c % CPK) * V * LS + c / CPK;
#pragma unroll
        for (int j = 0; j < V; ++j) d[j * LS] = e[j];
      }
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
  uint4 reg[NCH];
  __device__ void setup(int r0, int g) {
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
    }
  }
  __device__ void load(int k0) {
#pragma unroll
    for (int i = 0; i < NCH; ++i) {
      const int c = threadIdx.x + i * NTHREADS;
      const int k = k0 + (c % CPR) * V;
      uint4 v = make_uint4(0, 0, 0, 0);
      if (c < NCHUNK && k < K) {
        const int tap = k / cg.Cg, ci = k - tap * cg.Cg;
        const int kh = tap / cg.KW, kw = tap - kh * cg.KW;
        const int hi = hb[i] + kh, wi = wb[i] + kw;
        if ((unsigned)hi < (unsigned)cg.H && (unsigned)wi < (unsigned)cg.W)
          v = *reinterpret_cast<const uint4*>(rowp[i] + ((int64_t)hi * cg.W + wi) * cg.Ctot + ci);
      }
      reg[i] = v;
    }
  }
  __device__ void store(T* s) {
#pragma unroll
    for (int i = 0; i < NCH; ++i) {
      const int c = threadIdx.x + i * NTHREADS;
      if (c < NCHUNK) *reinterpret_cast<uint4*>(s + (c / CPR) * LS + (c % CPR) * V) = reg[i];
    }
  }
};

// Layer-1 input: NCHW images with three channels, stride 4, 11x11, no padding;
// k = (c, kh, kw) = the OIHW order of the layer-1 weights (363 values, zero
// beyond).  In ten-view mode image n is view n % 10 of source n / 10: the
// crop offset and mirroring are applied on the fly.
struct Conv1Src {
  int Hs, Ws;        // source plane size (227, or 256 for ten-view sources)
  int tenview;       // 0 or 1
  int crop;          // 227
};

__device__ __forceinline__ void tenview_offset(int v, int d, int& y0, int& x0, int& flip) {
  const int b = v % 5;
  y0 = (b == 2 || b == 3) ? d : (b == 4 ? d / 2 : 0);
  x0 = (b == 1 || b == 3) ? d : (b == 4 ? d / 2 : 0);
  flip = v >= 5;
}

template <typename T, int R>
struct LdConv1 {
  static constexpr int V = VecOf<T>::V, CPR = BK / V, NCHUNK = R * CPR;
  static constexpr int NCH = (NCHUNK + NTHREADS - 1) / NTHREADS;
  static constexpr int LS = Lds<T>::LS;
  static constexpr int KREAL = 3 * 11 * 11;
  const T* p; Conv1Src src; int M;
  const T* img[NCH]; int y[NCH], x[NCH], dir[NCH];
  uint4 reg[NCH];
  __device__ void setup(int r0, int) {
#pragma unroll
    for (int i = 0; i < NCH; ++i) {
      const int c = threadIdx.x + i * NTHREADS;
      const int m = r0 + c / CPR;
      img[i] = nullptr; y[i] = 0; x[i] = 0; dir[i] = 1;
      if (c < NCHUNK && m < M) {
        const int n = m / 3025, rem = m - n * 3025;
        const int ho = rem / 55, wo = rem - ho * 55;
        if (src.tenview) {
          int y0, x0, flip;
          tenview_offset(n % 10, src.Hs - src.crop, y0, x0, flip);
          img[i] = p + (int64_t)(n / 10) * 3 * src.Hs * src.Ws;
          y[i] = y0 + ho * 4;
          x[i] = flip ? x0 + src.crop - 1 - wo * 4 : x0 + wo * 4;
          dir[i] = flip ? -1 : 1;
        } else {
          img[i] = p + (int64_t)n * 3 * src.Hs * src.Ws;
          y[i] = ho * 4; x[i] = wo * 4;
        }
      }
    }
  }
  __device__ void load(int k0) {
#pragma unroll
    for (int i = 0; i < NCH; ++i) {
      const int c = threadIdx.x + i * NTHREADS;
      T e[V];
#pragma unroll
      for (int j = 0; j < V; ++j) {
        const int k = k0 + (c % CPR) * V + j;
        T val = T(0);
        if (c < NCHUNK && img[i] && k < KREAL) {
          const int ch = k / 121, r = k - ch * 121;
          const int kh = r / 11, kw = r - kh * 11;
          val = img[i][((int64_t)ch * src.Hs + y[i] + kh) * src.Ws + x[i] + dir[i] * kw];
        }
        e[j] = val;
      }
      reg[i] = pack_u4(e);
    }
  }
  __device__ void store(T* s) {
#pragma unroll
    for (int i = 0; i < NCH; ++i) {
      const int c = threadIdx.x + i * NTHREADS;
      if (c < NCHUNK) *reinterpret_cast<uint4*>(s + (c / CPR) * LS + (c % CPR) * V) = reg[i];
    }
  }
};

// Weight-gradient B operand: element (r = (kh, kw, ci), k = output pixel p) =
// X[n(p)][ho*s - pad + kh][wo*s - pad + kw][g*Cg + ci] of an NHWC tensor.
// k is outer, so the slice is transposed into LDS.  Needs Cg % V == 0.
template <typename T, int R>
struct LdWgradB {
  static constexpr int V = VecOf<T>::V, CPK = R / V, NCHUNK = BK * CPK;
  static constexpr int NCH = (NCHUNK + NTHREADS - 1) / NTHREADS;
  static constexpr int LS = Lds<T>::LS;
  const T* p; ConvGeom cg; int rows; int P;   // rows = KH*KW*Cg, P = Nimg*Ho*Wo
  int r0; const T* gbase;
  uint4 reg[NCH];
  __device__ void setup(int r0_, int g) { r0 = r0_; gbase = p + g * cg.Cg; }
  __device__ void load(int k0) {
#pragma unroll
    for (int i = 0; i < NCH; ++i) {
      const int c = threadIdx.x + i * NTHREADS;
      uint4 v = make_uint4(0, 0, 0, 0);
      const int pk = k0 + c / CPK, r = r0 + (c % CPK) * V;
      if (c < NCHUNK && pk < P && r < rows) {
        const int tap = r / cg.Cg, ci = r - tap * cg.Cg;
        const int kh = tap / cg.KW, kw = tap - kh * cg.KW;
        const int hw = cg.Ho * cg.Wo;
        const int n = pk / hw, rem = pk - n * hw;
        const int ho = rem / cg.Wo, wo = rem - ho * cg.Wo;
        const int hi = ho * cg.stride - cg.pad + kh, wi = wo * cg.stride - cg.pad + kw;
        if ((unsigned)hi < (unsigned)cg.H && (unsigned)wi < (unsigned)cg.W)
          v = *reinterpret_cast<const uint4*>(gbase + (((int64_t)n * cg.H + hi) * cg.W + wi) * cg.Ctot + ci);
      }
      reg[i] = v;
    }
  }
  __device__ void store(T* s) {
#pragma unroll
    for (int i = 0; i < NCH; ++i) {
      const int c = threadIdx.x + i * NTHREADS;
      if (c < NCHUNK) {
        T e[V];
        unpack_u4(reg[i], e);
        T* d = s + (c % CPK) * V * LS + c / CPK;
#pragma unroll
        for (int j = 0; j < V; ++j) d[j * LS] = e[j];
      }
    }
  }
};

// Layer-1 weight-gradient B operand: element (r = (c, kh, kw), k = output pixel)
// of the NCHW input images (scalar gathers; r beyond 363 reads as zero).
template <typename T, int R>
struct LdConv1WgradB {
  static constexpr int V = VecOf<T>::V, CPK = R / V, NCHUNK = BK * CPK;
  static constexpr int NCH = (NCHUNK + NTHREADS - 1) / NTHREADS;
  static constexpr int LS = Lds<T>::LS;
  const T* p; int Hs, Ws; int P;
  int r0;
  T reg[NCH][V];
  __device__ void setup(int r0_, int) { r0 = r0_; }
  __device__ void load(int k0) {
#pragma unroll
    for (int i = 0; i < NCH; ++i) {
      const int c = threadIdx.x + i * NTHREADS;
      const int pk = k0 + c / CPK, rb = r0 + (c % CPK) * V;
      const bool ok = c < NCHUNK && pk < P;
      int n = 0, ho = 0, wo = 0;
      if (ok) { n = pk / 3025; const int rem = pk - n * 3025; ho = rem / 55; wo = rem - ho * 55; }
      const T* img = p + (int64_t)n * 3 * Hs * Ws;
#pragma unroll
      for (int j = 0; j < V; ++j) {
        const int r = rb + j;
        T val = T(0);
        if (ok && r < 363) {
          const int ch = r / 121, q = r - ch * 121;
          const int kh = q / 11, kw = q - kh * 11;
          val = img[((int64_t)ch * Hs + ho * 4 + kh) * Ws + wo * 4 + kw];
        }
        reg[i][j] = val;
      }
    }
  }
  __device__ void store(T* s) {
#pragma unroll
    for (int i = 0; i < NCH; ++i) {
      const int c = threadIdx.x + i * NTHREADS;
      if (c < NCHUNK) {
        T* d = s + (c % CPK) * V * LS + c / CPK;
#pragma unroll
        for (int j = 0; j < V; ++j) d[j * LS] = reg[i][j];
      }
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
  static constexpr int LS = Lds<bf16>::LS;
  static __device__ __forceinline__ void run(const bf16* As, const bf16* Bs, f32x4_t (&acc)[FM][FN],
                                             int lane) {
    const int r = lane & 15, kq = (lane >> 4) * 8;
    bf16x8_t a[FM], b[FN];
#pragma unroll
    for (int i = 0; i < FM; ++i) a[i] = *reinterpret_cast<const bf16x8_t*>(As + (i * 16 + r) * LS + kq);
#pragma unroll
    for (int j = 0; j < FN; ++j) b[j] = *reinterpret_cast<const bf16x8_t*>(Bs + (j * 16 + r) * LS + kq);
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
      for (int j = 0; j < FN; ++j)
        acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[i], b[j], acc[i][j], 0, 0, 0);
  }
};

template <int FM, int FN>
struct Mma<float, FM, FN> {
  static constexpr int LS = Lds<float>::LS;
  static __device__ __forceinline__ void run(const float* As, const float* Bs, f32x4_t (&acc)[FM][FN],
                                             int lane) {
    const int r = lane & 15, kq = lane >> 4;
#pragma unroll
    for (int kk = 0; kk < BK; kk += 4) {
      float a[FM], b[FN];
#pragma unroll
      for (int i = 0; i < FM; ++i) a[i] = As[(i * 16 + r) * LS + kk + kq];
#pragma unroll
      for (int j = 0; j < FN; ++j) b[j] = Bs[(j * 16 + r) * LS + kk + kq];
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

  al.setup(m0, g);
  bl.setup(n0, g);
  f32x4_t acc[FM][FN];
#pragma unroll
  for (int i = 0; i < FM; ++i)
#pragma unroll
    for (int j = 0; j < FN; ++j) acc[i][j] = f32x4_t{0.f, 0.f, 0.f, 0.f};

  if (kt0 < kt1) {
    al.load(kt0 * BK);
    bl.load(kt0 * BK);
    al.store(As);
    bl.store(Bs);
    __syncthreads();
    for (int kt = kt0; kt < kt1; ++kt) {
      const int cur = (kt - kt0) & 1;
      const bool more = kt + 1 < kt1;
      if (more) { al.load((kt + 1) * BK); bl.load((kt + 1) * BK); }
      Mma<T, FM, FN>::run(As + cur * A_EL + wm * WTM * LS, Bs + cur * B_EL + wn * WTN * LS, acc, lane);
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
