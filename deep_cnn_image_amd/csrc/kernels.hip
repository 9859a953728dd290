// AlexNet kernels for gfx950 and their launchers.
//
// Dense contractions go through the MFMA GEMM core in gemm.hpp.  The rest are
// bandwidth-bound kernels over NHWC activations: each thread owns one pixel
// and a run of 8 consecutive channels, so every global access is a 16-byte
// (bf16) or 2x16-byte (fp32) vector access and a wavefront covers contiguous
// memory.
#include "common.hpp"
#include "gemm.hpp"
#include "launch.hpp"

namespace ax {

static constexpr int TPB = 256;

// k-contiguous operand loaders: direct-to-LDS for bf16, through registers for fp32
template <typename T, int R>
using RowsLd = std::conditional_t<std::is_same<T, bf16>::value, DmaKC<R>, LdKC<T, R>>;
template <typename T, int R>
using Im2colLd = std::conditional_t<std::is_same<T, bf16>::value, DmaIm2col<R>, LdIm2col<T, R>>;
// k-outer operand loaders: direct-to-LDS with transposing fragment reads for bf16
template <typename T, int R>
using ColsLd = std::conditional_t<std::is_same<T, bf16>::value, DmaKO<R>, LdKO<T, R>>;
template <typename T, int R>
using WgradBLd = std::conditional_t<std::is_same<T, bf16>::value, DmaWgradB<R>, LdWgradB<T, R>>;
// channel-blocked k order (direct-to-LDS im2col only; see DmaIm2col)
template <int R> static void set_blocked(DmaIm2col<R>& a, bool b) { a.blocked = b; }
template <typename T, int R> static void set_blocked(LdIm2col<T, R>&, bool) {}
// the direct-to-LDS im2col's per-row tap bits (see DmaIm2col) hold the geometry
template <int R> static bool im2col_fits(const DmaIm2col<R>& a) {
  return im2col_taps_fit(a.cg.KH, a.cg.KW, a.cg.Cg, a.blocked);
}
template <typename T, int R> static bool im2col_fits(const LdIm2col<T, R>&) { return true; }
bool im2col_blocked(DType dt, int Cg);

static inline dim3 grid1d(int64_t n) { return dim3((unsigned)((n + TPB - 1) / TPB)); }

static inline void rec_start(const KTimer* kt, hipStream_t st) { if (kt) hipEventRecord(kt->start, st); }
static inline void rec_stop(const KTimer* kt, hipStream_t st) { if (kt) hipEventRecord(kt->stop, st); }

// =========================================================================
// GEMM launches
// =========================================================================
// ST = 0: the tile's default LDS stages (for direct-to-LDS k-contiguous
// operands under the read-ahead schedule: three of A and two of B where they
// fit beside a second workgroup).
template <typename T, int BM, int BN, int WGM, int WGN, int ST0 = 0, class AL, class BL, class EP>
static hipError_t run_gemm(const AL& al, const BL& bl, const EP& ep, int M, int N, int K, int groups,
                           int splits, hipStream_t st, const KTimer* kt = nullptr, int strip_n = 0) {
  constexpr bool ASYM = ST0 == 0 && AL::DMA &&
                        gemm_read_ahead<typename AL::Layout, typename BL::Layout, BM / WGM / 16, BN / WGN / 16>() &&
                        gemm_a_stages<T, BM, BN>() == 3;
  constexpr int ST = ASYM ? 3 : ST0 ? ST0 : gemm_default_stages<T, BM, BN>();
  constexpr int STB = ASYM ? 2 : ST;
  GemmGrid gg;
  gg.M = M; gg.N = N; gg.K = K;
  gg.tiles_m = cdiv(M, BM);
  gg.tiles_n = cdiv(N, BN);
  const int ktiles = cdiv(K, BK);
  gg.splits = eff_splits(K, splits);
  gg.kt_per_split = cdiv(ktiles, gg.splits);
  gg.groups = groups;
  gg.strip_n = strip_n;
  dim3 grid(gg.tiles_m * gg.tiles_n * groups * gg.splits);
  rec_start(kt, st);
  hipLaunchKernelGGL((k_gemm<T, BM, BN, WGM, WGN, AL, BL, EP, ST, STB>), grid, dim3(NTHREADS), 0, st, al, bl,
                     ep, gg);
  rec_stop(kt, st);
  return hipGetLastError();
}

// ---- layer 1: space-to-depth
// The stride-4 11x11 convolution over 3 channels is evaluated as a stride-1
// 3x3 convolution over 4x4 pixel blocks: X'[n][bh][bw][c*16 + dh*4 + dw] =
// x[n][c][4bh+dh][4bw+dw] (zero beyond the 227x227 image), 57x57 blocks of 48
// values, and W'[co][kh'][kw'][c*16 + dh*4 + dw] = W[co][c][4kh'+dh][4kw'+dw]
// (zero where 4kh'+dh or 4kw'+dw >= 11).  Output (ho, wo) reads blocks
// (ho + kh', wo + kw'), i.e. pixels 4ho + kh, 4wo + kw: the same sum.
static constexpr int S2D_B = 57, S2D_C = 48, S2D_K = 3 * 3 * S2D_C;

__device__ __forceinline__ void tenview_offset(int v, int d, int& y0, int& x0, int& flip) {
  const int b = v % 5;
  y0 = (b == 2 || b == 3) ? d : (b == 4 ? d / 2 : 0);
  x0 = (b == 1 || b == 3) ? d : (b == 4 ? d / 2 : 0);
  flip = v >= 5;
}

// Training-time augmentation (ImageNet Classification with Deep
// Convolutional Neural Networks, section 4.1): the patch of source n and its
// mirror flag, and the RGB shift added to every pixel of the image, the
// principal components weighted by the image's draws alpha times the
// eigenvalues.  Crop offsets outside the source are clamped into it.
__device__ __forceinline__ void aug_patch(const AugSrc& a, int n, int Hs, int Ws, int& y0, int& x0, int& flip) {
  const int32_t* c = a.crop + 3 * n;
  y0 = min(max(c[0], 0), Hs - 227);
  x0 = min(max(c[1], 0), Ws - 227);
  flip = c[2] != 0;
}
__device__ __forceinline__ float aug_shift(const AugSrc& a, int n, int ch) {
  const float* al = a.alpha + 3 * n;
  const float* p = a.eigvec + 3 * ch;
  float s = p[0] * (al[0] * a.eigval[0]);
  s = fmaf(p[1], al[1] * a.eigval[1], s);
  s = fmaf(p[2], al[2] * a.eigval[2], s);
  return s;
}
// pixel value plus shift, rounded once to T
template <typename T>
__device__ __forceinline__ T aug_value(T v, float shift) { return Num<T>::store(Num<T>::load(v) + shift); }

// One workgroup per (image, block row).  The 12 input rows it needs (3
// channels x 4 rows) are copied into LDS as whole 16-byte chunks: image rows
// start at any element (227 is odd), so each row's copy begins at the chunk
// boundary below its first element and the row sits in LDS at that shift.
// The 57 x 48 values of the block row are then written as 16-byte runs.
// Ten-view sources: image n is view n % 10 of source n / 10 (227x227 crop at
// the view's offset, mirrored for views 5..9).  Augmented sources: image n is
// the patch of source n given by `aug`, with its RGB shift.  `total` is the
// element count of x; a chunk that would cross its end is read element by
// element.
template <typename T>
__device__ __forceinline__ void s2d_block(int blk, const T* __restrict__ x, T* __restrict__ xs, int Hs, int Ws,
                                          int kind, const AugSrc& aug, int64_t total) {
  constexpr int V = 16 / (int)sizeof(T);                // elements per chunk
  constexpr int RCH = (V + 225) / V + 1;                // chunks per staged row (span of 227 at shift < V)
  constexpr int RS = RCH * V;                           // LDS row stride, elements
  __shared__ __attribute__((aligned(16))) T rows[12 * RS];
  __shared__ int shift[12];
  const int n = blk / S2D_B, bh = blk - n * S2D_B;
  int y0 = 0, x0 = 0, flip = 0;
  int64_t img;
  float rgb[3] = {0.f, 0.f, 0.f};
  if (kind == SRC_TENVIEW) {
    tenview_offset(n % 10, Hs - 227, y0, x0, flip);
    img = (int64_t)(n / 10) * 3 * Hs * Ws;
  } else {
    if (kind == SRC_AUGMENT) {
      aug_patch(aug, n, Hs, Ws, y0, x0, flip);
#pragma unroll
      for (int c = 0; c < 3; ++c) rgb[c] = aug_shift(aug, n, c);
    }
    img = (int64_t)n * 3 * Hs * Ws;
  }
  for (int i = threadIdx.x; i < 12 * RCH; i += TPB) {
    const int r = i / RCH, ch = i - r * RCH;
    const int c = r >> 2, yc = 4 * bh + (r & 3);
    if (yc >= 227) continue;                             // below the image: never read
    const int64_t first = img + ((int64_t)c * Hs + y0 + yc) * Ws + x0;   // element of column 0
    const int64_t e0 = (first & ~(int64_t)(V - 1)) + (int64_t)ch * V;
    if (ch == 0) shift[r] = (int)(first & (V - 1));
    if (e0 > first + 226) continue;                      // past the row's last chunk
    uint4 q;
    if (e0 + V <= total) {
      q = *reinterpret_cast<const uint4*>(x + e0);
    } else {
      T e[V];
#pragma unroll
      for (int j = 0; j < V; ++j) e[j] = e0 + j < total ? x[e0 + j] : T(0);
      q = pack_u4(e);
    }
    *reinterpret_cast<uint4*>(rows + r * RS + ch * V) = q;
  }
  __syncthreads();
  // An output chunk holds V consecutive values c*16 + dh*4 + dw of one block:
  // one channel, V / 4 consecutive rows dh (two for bf16, one for fp32) and
  // the four columns of each, so row base, shift, direction and bounds are
  // worked out once per row rather than per value.
  static_assert(V % 4 == 0 && S2D_C % V == 0, "an output chunk spans whole 4-column runs");
  T* out = xs + (int64_t)blk * S2D_B * S2D_C;
  for (int i = threadIdx.x; i < S2D_B * S2D_C / V; i += TPB) {
    const int bw = (i * V) / S2D_C, q0 = i * V - bw * S2D_C;
    const int c = q0 >> 4, dh0 = (q0 >> 2) & 3;
    const int ncol = min(4, 227 - 4 * bw);   // columns inside the image
    float sh = 0.f;
    if (kind == SRC_AUGMENT) sh = c == 0 ? rgb[0] : c == 1 ? rgb[1] : rgb[2];
    T e[V];
#pragma unroll
    for (int h = 0; h < V / 4; ++h) {
      const int dh = dh0 + h, r = c * 4 + dh;
      const bool rowok = 4 * bh + dh < 227;
      // column xc of the view is at p[dw * stp]: xc = 4 bw + dw, mirrored 226 - xc
      const T* p = rows + r * RS + shift[r] + (flip ? 226 - 4 * bw : 4 * bw);
      const int stp = flip ? -1 : 1;
#pragma unroll
      for (int dw = 0; dw < 4; ++dw) {
        T v = T(0);
        if (rowok && dw < ncol) {
          v = p[dw * stp];
          if (kind == SRC_AUGMENT) v = aug_value(v, sh);
        }
        e[h * 4 + dw] = v;
      }
    }
    *reinterpret_cast<uint4*>(out + i * V) = pack_u4(e);
  }
}

// Tile for an implicit-GEMM convolution with M output rows, N columns per
// group.  n-tile: 128 when it divides N, else 96, else 48 (four waves stacked
// along m), else 128 with a ragged last tile.  m-tile (bf16): the one of 96,
// 128, 192 whose tiles finish in the fewest rounds of the 512 workgroups the
// chip holds at once (two per CU), weighted slightly towards taller tiles,
// which reuse each B slice over more rows.
constexpr int RESIDENT_WG = 512;
static int pick_bm(int M, int N, int BN, int groups) {
  const int cand[3] = {96, 128, 192};
  const float weight[3] = {1.10f, 1.0f, 0.95f};
  int best = 128;
  float best_cost = 3.0e38f;
  for (int i = 0; i < 3; ++i) {
    const int64_t tiles = (int64_t)cdiv(M, cand[i]) * cdiv(N, BN) * groups;
    const float cost = (float)((tiles + RESIDENT_WG - 1) / RESIDENT_WG) * cand[i] * weight[i];
    if (cost < best_cost) { best_cost = cost; best = cand[i]; }
  }
  return best;
}

template <int BN, class Fn>
static hipError_t by_bm(int bm, Fn&& fn) {
  switch (bm) {
    case 96: return fn.template operator()<96, BN, 2, 2>();
    case 192: return fn.template operator()<192, BN, 2, 2>();
    default: return fn.template operator()<128, BN, 2, 2>();
  }
}

// Tile (BM x BN) that by_tile runs for an M x N (per group) convolution GEMM.
static void conv_tile(bool bf, int M, int N, int groups, int& bm, int& bn) {
  const bool bn128 = N % 128 == 0 || (N % 96 != 0 && !(N % 48 == 0 && N <= 96));
  bn = bn128 ? 128 : N % 96 == 0 ? 96 : 48;
  bm = bf && bn != 48 ? pick_bm(M, N, bn, groups) : 128;
}

template <typename T, class Fn>
static hipError_t by_tile(int M, int N, int groups, Fn&& fn) {
  int bm, bn;
  conv_tile(std::is_same<T, bf16>::value, M, N, groups, bm, bn);
  if constexpr (std::is_same<T, bf16>::value) {
    if (bn == 128) return by_bm<128>(bm, fn);
    if (bn == 96) return by_bm<96>(bm, fn);
  } else {
    if (bn == 128) return fn.template operator()<128, 128, 2, 2>();
    if (bn == 96) return fn.template operator()<128, 96, 2, 2>();
  }
  return fn.template operator()<128, 48, 4, 1>();
}

// ---- split-K for convolutions too small to fill the chip (small batches)
// With fewer workgroups than CUs, each one's long k loop is the whole run
// time.  The k range is then split until the chip holds one round of
// workgroups (512 bf16 ones, two per CU; 256 fp32 ones, whose LDS tiles
// allow one per CU), each over at least three k-slices for bf16 or one for
// fp32 (whose slices carry 16 times the matrix-core time).  fp32 partials go
// to the workspace and k_fc_reduce sums them in split order and applies the
// epilogue (bias and ReLU forward, the ReLU mask for a data gradient).  At
// batch 128 every layer's tiles alone fill the chip and nothing is split.
static int conv_split_count(int64_t wgs, int K, bool f32) {
  if (wgs >= 256) return 1;
  const int kt = cdiv(K, GEMM_BK);
  int want = (int)(((f32 ? 256 : 512) + wgs - 1) / wgs);
  const int cap = f32 ? kt : kt / 3;
  if (want > cap) want = cap;
  return eff_splits(K, want);
}

static int conv_gemm_splits(DType dt, int M, int N, int K, int groups) {
  int bm, bn;
  conv_tile(dt == BF16, M, N, groups, bm, bn);
  return conv_split_count((int64_t)cdiv(M, bm) * cdiv(N, bn) * groups, K, dt == F32);
}

template <typename T>
__global__ void k_fc_reduce(const float* __restrict__ part, int S, int M, int N, int64_t ldo,
                            const T* __restrict__ bias, FcEpi ep, const T* __restrict__ mask, T* __restrict__ out,
                            float* __restrict__ out_f32);

// Partials part[g][s][m][n] (n < N per group), then per group the ordered
// sum into out[m * ldo + g * N + n]: forward with bias (bias[g * N + n]) and
// ReLU; data gradient with the mask [mask > 0] (mask laid out as out).
template <typename T, int BM, int BN, int WGM, int WGN, class AL, class BL>
static hipError_t conv_split_k(const AL& a, const BL& b, int M, int N, int K, int groups, int S,
                               const void* bias, bool relu, const void* mask, void* y, int64_t ldo, float* part,
                               size_t part_bytes, hipStream_t st, const KTimer* kt) {
  if (N % 4 || (size_t)S * groups * M * N * sizeof(float) > part_bytes) return hipErrorInvalidValue;
  EpF32 e;
  e.out = part; e.ldo = N; e.M = M; e.N = N; e.splits = S;
  rec_start(kt, st);
  hipError_t err = run_gemm<T, BM, BN, WGM, WGN>(a, b, e, M, N, K, groups, S, st);
  if (err != hipSuccess) return err;
  FcEpi ep{};
  ep.relu = relu ? 1 : 0;
  for (int g = 0; g < groups; ++g)
    hipLaunchKernelGGL((k_fc_reduce<T>), grid1d((int64_t)M * N / 4), dim3(TPB), 0, st,
                       part + (size_t)g * S * M * N, S, M, N, ldo, bias ? (const T*)bias + g * N : nullptr, ep,
                       mask ? (const T*)mask + g * N : nullptr, (T*)y + g * N, (float*)nullptr);
  rec_stop(kt, st);
  return hipGetLastError();
}

static ConvGeom conv1_geom() { return ConvGeom{S2D_B, S2D_B, S2D_C, S2D_C, 3, 3, 1, 0, 55, 55}; }

template <typename T>
struct Conv1FwdFn {
  const void* xs; int Nimg; const void* ws2d; const void* b1; void* y; float* part; size_t part_bytes;
  hipStream_t st; const KTimer* kt;
  template <int BM, int BN, int WGM, int WGN>
  hipError_t operator()() const {
    Im2colLd<T, BM> a;
    a.p = (const T*)xs; a.cg = conv1_geom(); a.M = Nimg * 3025; a.K = S2D_K;
    if (!im2col_fits(a)) return hipErrorInvalidValue;
    RowsLd<T, BN> b;
    b.p = (const T*)ws2d; b.ld = S2D_K; b.rows = 96; b.K = S2D_K; b.gstride = 0;
    const int S = conv_split_count(cdiv(a.M, BM) * cdiv(96, BN), S2D_K, std::is_same<T, float>::value);
    if (S > 1) return conv_split_k<T, BM, BN, WGM, WGN>(a, b, a.M, 96, S2D_K, 1, S, b1, true, nullptr, y, 96, part,
                                                        part_bytes, st, kt);
    EpBiasRelu<T> e;
    e.out = (T*)y; e.bias = (const T*)b1; e.ldo = 96; e.M = a.M; e.N = 96;
    return run_gemm<T, BM, BN, WGM, WGN>(a, b, e, a.M, 96, S2D_K, 1, 1, st, kt);
  }
};

// ---- layer 1 forward, bf16: direct convolution over block rows kept in LDS
// In the space-to-depth form layer 1 has K = 432 (9 taps x 48 values) per
// output and 96 outputs per pixel.  An implicit-GEMM workgroup would run only
// 7 k-slices, so filling and draining its pipeline takes much of its life, and
// it would gather each input block once per tap.  Here one workgroup per CU
// stays resident, with W' in LDS for the whole launch.  It walks tiles of 4
// output rows x 55 columns (220 pixels) of one image.  A tile's 6 input block
// rows (96 bytes per block) are copied into LDS with direct-to-LDS loads, into
// one of two buffers while the previous tile is multiplied from the other.
// Rows of 96 bytes (W' rows of 864) keep the fragment reads free of bank
// conflicts: a 16-byte LDS read serves 32 lanes at a time over 128 banks, and
// 16 rows at that stride, with the next 16 lanes 16 bytes further on, touch
// every bank once (rows of 112 or 144 bytes conflict two-way).  Eight
// waves (two per SIMD) each take 48 channels and a quarter of the tile's
// pixels.  Each product takes the weights as the first MFMA operand (16
// channels x 32 k) and the block rows as the second (32 k x 16 pixels), so a
// lane ends with 4 consecutive channels of one pixel.  The first product of a
// tile starts from the bias instead of zero; ReLU and rounding are applied in
// registers.  The next tile's loads and this tile's 8-byte output runs are
// issued between the products, a few per k-step, instead of in bursts that
// every CU would issue at the same moment.  k runs in the same order as in the
// implicit GEMM, 32 at a time; in the 14th step's upper half (k >= 432) the
// weight fragment is zero (and the block-row fragment any finite data).
constexpr int C1_ROWS = 4;                               // output rows per tile
constexpr int C1_TPI = (55 + C1_ROWS - 1) / C1_ROWS;     // tiles per image
constexpr int C1_PROWS = C1_ROWS + 2;                    // input block rows per tile
constexpr int C1_SLOT = S2D_C / 8;                       // 16-byte granules per block
constexpr int C1_GRAN = C1_PROWS * S2D_B * C1_SLOT;      // granules per tile
constexpr int C1_NI = (C1_GRAN + 63) / 64;               // direct-to-LDS loads per tile (1 KB each)
constexpr int C1_WAVES = 8;                              // two per SIMD
constexpr int C1_NIW = (C1_NI + C1_WAVES - 1) / C1_WAVES;   // per wave, at most
constexpr int C1_BUF = C1_NI * 64 * 8;                   // bf16 elements per block-row buffer
constexpr int C1_KS = (S2D_K + 31) / 32;                 // k-steps of 32
constexpr int C1_FM = 4, C1_FN = 3;                      // per wave: up to 4 x 16 pixels, 3 x 16 channels
constexpr int C1_WL = (int)(S2D_W_ELEMS * 2 / 1024);     // direct-to-LDS loads of W' (1 KB each)
constexpr int C1_GRID = 256;                             // one workgroup per CU
static_assert(C1_ROWS * 55 <= 224 && 2 * C1_FN * 16 == 96, "eight waves cover a tile: m-fragments 4, 4, 3, 3");
static_assert(S2D_C % 8 == 0 && S2D_K % 8 == 0, "an 8-value k run stays within one tap");
static_assert(C1_NIW <= C1_KS && C1_FM <= C1_KS, "one load and one row of stores per k-step at most");
static_assert(S2D_W_ELEMS * 2 % 1024 == 0 && (2 * C1_BUF + C1_WL * 512) * 2 <= 160 * 1024, "block rows and W' fit in LDS");
static_assert(((C1_PROWS - 1) * S2D_B + S2D_B - 1) * S2D_C * 2 + S2D_C * 2 < 65536, "block offsets fit 16 bits");

__global__ void __launch_bounds__(64 * C1_WAVES) __attribute__((amdgpu_waves_per_eu(2, 2)))
k_conv1_fwd(const bf16* __restrict__ xs, const bf16* __restrict__ w, const bf16* __restrict__ bias,
            bf16* __restrict__ y, int Nimg) {
  // [block rows 0][block rows 1][W' [96][432]]
  __shared__ __attribute__((aligned(16))) bf16 lds[2 * C1_BUF + C1_WL * 512];
  const bf16* const wl = lds + 2 * C1_BUF;
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int wn = wave & 1, wm = wave >> 1;
  // this wave's m-fragments: 4 from fragment 4 wm (wm < 2), else 3 from 8 + 3 (wm - 2)
  const int mf0 = wm < 2 ? 4 * wm : 8 + 3 * (wm - 2);
  const bool full = wm < 2;
  // Workgroups are dealt round-robin over the eight XCDs; XCD x takes a
  // contiguous run of the tile order, so that neighbouring tiles, which share
  // two block rows, share an L2.
  const int tiles = Nimg * C1_TPI;
  const int x = blockIdx.x & 7, per_x = gridDim.x >> 3;
  const int tq = tiles >> 3, tr = tiles & 7;
  const int t_end = x * tq + min(x, tr) + tq + (x < tr ? 1 : 0);
  int t = x * tq + min(x, tr) + (blockIdx.x >> 3);
  if (t >= t_end) return;

  const __amdgpu_buffer_rsrc_t rs = buf_rsrc(xs, (uint32_t)((int64_t)Nimg * S2D_ELEMS * 2));
  // Load i of this wave (j = wave + C1_WAVES i) copies granules 64 j .. 64 j
  // + 63 of the tile's block rows, which are contiguous in memory.  This
  // lane's granule lies in block row `row` of the tile, packed as (row << 16)
  // | byte offset, or past the tile (row 0xFFFF): loaded as zero.
  uint32_t drel[C1_NIW];
#pragma unroll
  for (int i = 0; i < C1_NIW; ++i) {
    const int gidx = (wave + C1_WAVES * i) * 64 + lane;
    const int row = gidx / (S2D_B * C1_SLOT);
    drel[i] = gidx < C1_GRAN ? ((uint32_t)row << 16) | (uint32_t)(gidx * 16) : 0xFFFF0000u;
  }
  auto dma = [&](int i, uint32_t base, int r0, bf16* buf) {
    const int j = wave + C1_WAVES * i;
    if (j < C1_NI) {
      const uint32_t d = drel[i];
      const uint32_t off = (int)(d >> 16) + r0 < S2D_B ? base + (d & 0xFFFFu) : BUF_OOB;
      dma16(rs, off, buf + j * 64 * 8);
    }
  };
  auto tile_base = [](int tile, int& r0) {
    const int n = tile / C1_TPI;
    r0 = (tile - n * C1_TPI) * C1_ROWS;
    return (uint32_t)(((int64_t)n * S2D_B + r0) * S2D_B * S2D_C * 2);
  };
  {
    int r0;
    const uint32_t base = tile_base(t, r0);
#pragma unroll
    for (int i = 0; i < C1_NIW; ++i) dma(i, base, r0, lds);
    // W' [96][432] as it is in memory
    const __amdgpu_buffer_rsrc_t rw = buf_rsrc(w, (uint32_t)(S2D_W_ELEMS * 2));
    for (int j = wave; j < C1_WL; j += C1_WAVES) dma16(rw, (uint32_t)(j * 1024 + lane * 16), lds + 2 * C1_BUF + j * 512);
  }

  // this lane's 4 output channels per n-fragment, and their biases as the
  // accumulator a tile's first product starts from
  const int c0 = wn * 48 + (lane >> 4) * 4;
  f32x4_t bc[C1_FN];
#pragma unroll
  for (int j = 0; j < C1_FN; ++j)
    bc[j] = f32x4_t{bf2f(bias[c0 + j * 16]), bf2f(bias[c0 + j * 16 + 1]), bf2f(bias[c0 + j * 16 + 2]),
                    bf2f(bias[c0 + j * 16 + 3])};
  // LDS element offsets: of the pixel's top-left block per m-fragment, of the
  // tap and channel run per k-step; of the weight row per n-fragment
  int poff[C1_FM];
#pragma unroll
  for (int i = 0; i < C1_FM; ++i) {
    const int px = min((mf0 + i) * 16 + (lane & 15), C1_ROWS * 55 - 1);
    const int lr = px / 55;
    poff[i] = (lr * S2D_B + px - lr * 55) * C1_SLOT * 8;
  }
  int woff[C1_FN];
#pragma unroll
  for (int j = 0; j < C1_FN; ++j) woff[j] = (wn * 48 + j * 16 + (lane & 15)) * S2D_K;
  auto toff = [&](int s) {
    const int k = min(s * 32 + (lane >> 4) * 8, S2D_K - 8);   // past K: any data (its weights are zero)
    const int tap = k / S2D_C, ci = k - tap * S2D_C, kh = tap / 3, kw = tap - kh * 3;
    return (kh * S2D_B + kw) * C1_SLOT * 8 + ci;
  };

  // the previous tile's outputs, rounded, stored during this tile's k-steps
  uint2 outv[C1_FM][C1_FN];
  bf16* yprev = nullptr;
  int npx_prev = 0;
  auto store_row = [&](int i, int j) {
    const int px = (mf0 + i) * 16 + (lane & 15);
    if ((i < C1_FM - 1 || full) && px < npx_prev) *reinterpret_cast<uint2*>(yprev + (int64_t)px * 96 + j * 16) = outv[i][j];
  };

  for (int it = 0;; ++it) {
    const bf16* cur = lds + (it & 1) * C1_BUF;
    bf16* nxt = lds + ((it + 1) & 1) * C1_BUF;
    wait_vmcnt<0>();
    lds_barrier();   // tile t's block rows (and at first W') are in; every wave is done with the other buffer
    const int tn = t + per_x;
    const bool more = tn < t_end;
    int nr0 = 0;
    const uint32_t nbase = more ? tile_base(tn, nr0) : 0u;
    const bool stores = yprev != nullptr;

    f32x4_t acc[C1_FM][C1_FN];
    bf16x8_t a[2][C1_FM], b[2][C1_FN];
    auto read = [&](int s, int buf) {
      const int to = toff(s), kr = s * 32 + (lane >> 4) * 8;
#pragma unroll
      for (int i = 0; i < C1_FM; ++i)
        if (i < C1_FM - 1 || full) a[buf][i] = *reinterpret_cast<const bf16x8_t*>(cur + poff[i] + to);
#pragma unroll
      for (int j = 0; j < C1_FN; ++j) {
        const bf16x8_t v = *reinterpret_cast<const bf16x8_t*>(wl + woff[j] + min(kr, S2D_K - 8));
        b[buf][j] = (s + 1) * 32 <= S2D_K || kr < S2D_K ? v : __builtin_bit_cast(bf16x8_t, make_uint4(0u, 0u, 0u, 0u));
      }
    };
    read(0, 0);
    // the next k-step's fragments are read before this one's products
#pragma unroll
    for (int s = 0; s < C1_KS; ++s) {
      if (s + 1 < C1_KS) read(s + 1, (s + 1) & 1);
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int i = 0; i < C1_FM; ++i) {
        if (i < C1_FM - 1 || full) {
#pragma unroll
          for (int j = 0; j < C1_FN; ++j)
            acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(b[s & 1][j], a[s & 1][i], s == 0 ? bc[j] : acc[i][j],
                                                                0, 0, 0);
        }
        if (i == 0 && s < C1_NIW && more) dma(s, nbase, nr0, nxt);
        if (i >= 1 && i <= C1_FN && s < C1_FM && stores) store_row(s, i - 1);
        __builtin_amdgcn_sched_barrier(0);
      }
    }

    const int n = t / C1_TPI, r0 = (t - n * C1_TPI) * C1_ROWS;
    npx_prev = min(C1_ROWS, 55 - r0) * 55;
    yprev = y + ((int64_t)n * 3025 + r0 * 55) * 96 + c0;
#pragma unroll
    for (int i = 0; i < C1_FM; ++i)
#pragma unroll
      for (int j = 0; j < C1_FN; ++j) {
        const f32x4_t u = acc[i][j];
        outv[i][j] = make_uint2(f2bf2(u[0] > 0.f ? u[0] : 0.f, u[1] > 0.f ? u[1] : 0.f),
                                f2bf2(u[2] > 0.f ? u[2] : 0.f, u[3] > 0.f ? u[3] : 0.f));
      }
    t = tn;
    if (!more) break;
  }
#pragma unroll
  for (int i = 0; i < C1_FM; ++i)
#pragma unroll
    for (int j = 0; j < C1_FN; ++j) store_row(i, j);
}

static hipError_t conv1_fwd_direct(const void* xs, int Nimg, const void* ws2d, const void* b1, void* y,
                                   hipStream_t st, const KTimer* kt) {
  // byte offsets into the staged input are 32-bit, below the out-of-range marker
  if (Nimg < 1 || (int64_t)Nimg * S2D_ELEMS * 2 >= (int64_t)BUF_OOB) return hipErrorInvalidValue;
  rec_start(kt, st);
  hipLaunchKernelGGL(k_conv1_fwd, dim3(C1_GRID), dim3(64 * C1_WAVES), 0, st, (const bf16*)xs, (const bf16*)ws2d,
                     (const bf16*)b1, (bf16*)y, Nimg);
  rec_stop(kt, st);
  return hipGetLastError();
}

template <typename T>
static hipError_t conv1_fwd_t(const void* xs, int Nimg, const void* ws2d, const void* b1, void* y, float* part,
                              size_t part_bytes, hipStream_t st, const KTimer* kt) {
  if constexpr (std::is_same<T, bf16>::value) return conv1_fwd_direct(xs, Nimg, ws2d, b1, y, st, kt);
  return by_tile<T>(Nimg * 3025, 96, 1, Conv1FwdFn<T>{xs, Nimg, ws2d, b1, y, part, part_bytes, st, kt});
}

hipError_t conv1_fwd(DType dt, const void* xs, int Nimg, const void* ws2d, const void* b1, void* y, float* part,
                     size_t part_bytes, hipStream_t st, const KTimer* kt) {
  return dt == BF16 ? conv1_fwd_t<bf16>(xs, Nimg, ws2d, b1, y, part, part_bytes, st, kt)
                    : conv1_fwd_t<float>(xs, Nimg, ws2d, b1, y, part, part_bytes, st, kt);
}

template <typename T>
struct ConvFwdFn {
  ConvShape s; const void* x; const void* wr; const void* b; void* y; float* part; size_t part_bytes;
  hipStream_t st; const KTimer* kt;
  template <int BM, int BN, int WGM, int WGN>
  hipError_t operator()() const {
    const int Cig = s.Cin / s.groups, Cog = s.Cout / s.groups;
    Im2colLd<T, BM> a;
    set_blocked(a, im2col_blocked(std::is_same<T, bf16>::value ? BF16 : F32, Cig));
    a.p = (const T*)x;
    a.cg = ConvGeom{s.H, s.W, s.Cin, Cig, s.K, s.K, s.stride, s.pad, s.Ho, s.Wo};
    a.M = s.Nimg * s.Ho * s.Wo;
    a.K = s.K * s.K * Cig;
    if (!im2col_fits(a)) return hipErrorInvalidValue;
    RowsLd<T, BN> bl;
    bl.p = (const T*)wr; bl.ld = a.K; bl.rows = Cog; bl.K = a.K; bl.gstride = (int64_t)Cog * a.K;
    const int S = conv_split_count((int64_t)cdiv(a.M, BM) * cdiv(Cog, BN) * s.groups, a.K,
                                   std::is_same<T, float>::value);
    if (S > 1)
      return conv_split_k<T, BM, BN, WGM, WGN>(a, bl, a.M, Cog, a.K, s.groups, S, b, true, nullptr, y, s.Cout,
                                               part, part_bytes, st, kt);
    EpBiasRelu<T> e;
    e.out = (T*)y; e.bias = (const T*)b; e.ldo = s.Cout; e.M = a.M; e.N = Cog;
    return run_gemm<T, BM, BN, WGM, WGN>(a, bl, e, a.M, Cog, a.K, s.groups, 1, st, kt);
  }
};

hipError_t conv_fwd(DType dt, const ConvShape& s, const void* x, const void* wr, const void* b, void* y,
                    float* part, size_t part_bytes, hipStream_t st, const KTimer* kt) {
  const int Cog = s.Cout / s.groups;
  const int M = s.Nimg * s.Ho * s.Wo;
  if (dt == BF16) {
    ConvFwdFn<bf16> f{s, x, wr, b, y, part, part_bytes, st, kt};
    return by_tile<bf16>(M, Cog, s.groups, f);
  }
  ConvFwdFn<float> f{s, x, wr, b, y, part, part_bytes, st, kt};
  return by_tile<float>(M, Cog, s.groups, f);
}

size_t conv_fwd_part_bytes(DType dt, const ConvShape& s) {
  const int Cog = s.Cout / s.groups, M = s.Nimg * s.Ho * s.Wo, K = s.K * s.K * (s.Cin / s.groups);
  const int S = conv_gemm_splits(dt, M, Cog, K, s.groups);
  return S > 1 ? (size_t)S * s.groups * M * Cog * sizeof(float) : 0;
}
size_t conv1_fwd_part_bytes(DType dt, int Nimg) {
  if (dt == BF16) return 0;   // k_conv1_fwd: no split
  const int S = conv_gemm_splits(dt, Nimg * 3025, 96, S2D_K, 1);
  return S > 1 ? (size_t)S * Nimg * 3025 * 96 * sizeof(float) : 0;
}

template <typename T>
struct ConvDgradFn {
  ConvShape s; const void* dy; const void* wt; const void* mask; void* dx; float* part; size_t part_bytes;
  hipStream_t st; const KTimer* kt;
  template <int BM, int BN, int WGM, int WGN>
  hipError_t operator()() const {
    const int Cig = s.Cin / s.groups, Cog = s.Cout / s.groups;
    // dX = stride-1 convolution of dY with flipped, transposed weights, pad K-1-p
    Im2colLd<T, BM> a;
    set_blocked(a, im2col_blocked(std::is_same<T, bf16>::value ? BF16 : F32, Cog));
    a.p = (const T*)dy;
    a.cg = ConvGeom{s.Ho, s.Wo, s.Cout, Cog, s.K, s.K, 1, s.K - 1 - s.pad, s.H, s.W};
    a.M = s.Nimg * s.H * s.W;
    a.K = s.K * s.K * Cog;
    if (!im2col_fits(a)) return hipErrorInvalidValue;
    RowsLd<T, BN> bl;
    bl.p = (const T*)wt; bl.ld = a.K; bl.rows = Cig; bl.K = a.K; bl.gstride = (int64_t)Cig * a.K;
    const int S = conv_split_count((int64_t)cdiv(a.M, BM) * cdiv(Cig, BN) * s.groups, a.K,
                                   std::is_same<T, float>::value);
    if (S > 1)
      return conv_split_k<T, BM, BN, WGM, WGN>(a, bl, a.M, Cig, a.K, s.groups, S, nullptr, false, mask, dx, s.Cin,
                                               part, part_bytes, st, kt);
    EpMask<T> e;
    e.out = (T*)dx; e.mask = (const T*)mask; e.ldo = s.Cin; e.M = a.M; e.N = Cig;
    return run_gemm<T, BM, BN, WGM, WGN>(a, bl, e, a.M, Cig, a.K, s.groups, 1, st, kt);
  }
};

hipError_t conv_dgrad(DType dt, const ConvShape& s, const void* dy, const void* wt, const void* mask,
                      void* dx, float* part, size_t part_bytes, hipStream_t st, const KTimer* kt) {
  if (s.stride != 1) return hipErrorInvalidValue;
  const int Cig = s.Cin / s.groups;
  const int M = s.Nimg * s.H * s.W;
  if (dt == BF16) {
    ConvDgradFn<bf16> f{s, dy, wt, mask, dx, part, part_bytes, st, kt};
    return by_tile<bf16>(M, Cig, s.groups, f);
  }
  ConvDgradFn<float> f{s, dy, wt, mask, dx, part, part_bytes, st, kt};
  return by_tile<float>(M, Cig, s.groups, f);
}

size_t conv_dgrad_part_bytes(DType dt, const ConvShape& s) {
  const int Cig = s.Cin / s.groups, M = s.Nimg * s.H * s.W, K = s.K * s.K * (s.Cout / s.groups);
  const int S = conv_gemm_splits(dt, M, Cig, K, s.groups);
  return S > 1 ? (size_t)S * s.groups * M * Cig * sizeof(float) : 0;
}

// ---- weight gradients: split-K partials, then an ordered reduction
// Enough splits to fill the chip once at two resident workgroups per CU, and
// never more than that: a few workgroups beyond it would cost a second round.
static int wgrad_splits(int tiles, int K) {
  int want = (2 * 256) / tiles;
  if (want > 256) want = 256;
  return eff_splits(K, want);
}

size_t conv_wgrad_part_bytes(const ConvShape& s) {
  const int Cig = s.Cin / s.groups, Cog = s.Cout / s.groups;
  const int N = s.K * s.K * Cig, P = s.Nimg * s.Ho * s.Wo;
  const int tiles = cdiv(Cog, 128) * cdiv(N, 128) * s.groups;
  return (size_t)s.groups * wgrad_splits(tiles, P) * Cog * N * sizeof(float);
}
static int64_t conv1_wgrad_direct_splits(int Nimg);
size_t conv1_wgrad_part_bytes(DType dt, int Nimg) {
  if (dt == BF16) return (size_t)conv1_wgrad_direct_splits(Nimg) * 96 * S2D_K * sizeof(float);
  const int tiles = cdiv(96, 128) * cdiv(S2D_K, 128);
  return (size_t)wgrad_splits(tiles, Nimg * 3025) * 96 * S2D_K * sizeof(float);
}

// gw[co][ci][kh][kw] = sum over the S split partials part[g][s][col][r], with
// co = g*Mg + col and
//   r = (kh*KW + kw)*Cg + ci                                  (mode 1)
//   r = ((kh/4)*3 + kw/4)*48 + ci*16 + (kh%4)*4 + kw%4        (mode 2: layer 1, space-to-depth;
//                                                               r outside the 11x11 taps is dropped)
// followed, when w is not null, by the SGD update of those weights: fp32
// master w and momentum v in place, working copy wb (the same element update
// as every other SGD path).
//
// Mode 1, k_wgrad_finish: one workgroup (16 waves) per output channel co.  It sums the S
// partial rows of co (Np = KH*KW*Cg values each, 16-byte loads, splits in
// order) into an LDS row, then walks the channel's OIHW slice in order, so
// the gradient, w, v and wb are read and written contiguously.
constexpr int WF_TPB = 1024;   // 16 waves per output channel keep enough loads in flight
template <typename T>
__global__ void __launch_bounds__(WF_TPB) k_wgrad_finish(const float* __restrict__ part, int S, int Mg, int Np,
                                                      int Cg, int KH, int KW, float* __restrict__ gw,
                                                      float* __restrict__ w, float* __restrict__ v,
                                                      T* __restrict__ wb, float lr, float mom, float wdlr) {
  extern __shared__ float4 row4[];
  float* row = reinterpret_cast<float*>(row4);
  const int co = blockIdx.x, g = co / Mg, col = co - g * Mg;
  const float4* p = reinterpret_cast<const float4*>(part + ((int64_t)g * S * Mg + col) * Np);
  const int64_t ss4 = (int64_t)Mg * Np / 4;
  for (int q = threadIdx.x; q < Np / 4; q += WF_TPB) {
    float4 acc = p[q];
#pragma unroll 4
    for (int s = 1; s < S; ++s) {
      const float4 x = p[s * ss4 + q];
      acc.x += x.x; acc.y += x.y; acc.z += x.z; acc.w += x.w;
    }
    row4[q] = acc;
  }
  __syncthreads();
  const int taps = KH * KW;
  const int64_t base = (int64_t)co * Np;   // OIHW slice of co (Cg*KH*KW == Np)
  for (int o = threadIdx.x; o < Np; o += WF_TPB) {
    const int ci = o / taps, t = o - ci * taps;
    const float gv = row[t * Cg + ci];      // (kh*KW + kw)*Cg + ci with t = kh*KW + kw
    gw[base + o] = gv;
    if (w) {
      float ww = w[base + o], vv = v[base + o];
      sgd_elem(ww, vv, gv, mom, wdlr, lr);
      w[base + o] = ww;
      v[base + o] = vv;
      wb[base + o] = Num<T>::store(ww);
    }
  }
}

// Mode 2 (layer 1: 96 channels, many splits), k_wgrad_reduce: a block covers
// 32 runs of four consecutive r (16-byte coalesced loads along the partial
// rows) with 8 split groups: group j sums splits j, j+8, ... in order, then
// the 8 group sums are added in order of j.  Needs Np % 4 == 0.
constexpr int WR_Q = 32, WR_G = TPB / WR_Q;
template <typename T>
__global__ void __launch_bounds__(TPB) k_wgrad_reduce(const float* __restrict__ part, int G, int S, int Mg,
                                                      int Np, int Cg, int KH, int KW, int mode,
                                                      float* __restrict__ gw, float* __restrict__ w,
                                                      float* __restrict__ v, T* __restrict__ wb, float lr,
                                                      float mom, float wdlr) {
  __shared__ float4 red[WR_G][WR_Q];
  const int qd = threadIdx.x % WR_Q, j = threadIdx.x / WR_Q;
  const int64_t t = (int64_t)blockIdx.x * WR_Q + qd;
  const int np4 = Np >> 2;
  const bool live = t < (int64_t)G * Mg * np4;
  const int co = live ? (int)(t / np4) : 0;
  const int r0 = live ? (int)(t - (int64_t)co * np4) * 4 : 0;
  const int g = co / Mg, col = co - g * Mg;
  float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
  if (live) {
    const float* p = part + ((int64_t)g * S * Mg + col) * Np + r0;
    const int64_t ss = (int64_t)Mg * Np;
    // eight loads in flight; the adds stay in split order
#pragma unroll 8
    for (int s = j; s < S; s += WR_G) {
      const float4 q = *reinterpret_cast<const float4*>(p + s * ss);
      acc.x += q.x; acc.y += q.y; acc.z += q.z; acc.w += q.w;
    }
  }
  red[j][qd] = acc;
  __syncthreads();
  if (j != 0 || !live) return;
  float a[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int jj = 0; jj < WR_G; ++jj) {
    const float4 q = red[jj][qd];
    a[0] += q.x; a[1] += q.y; a[2] += q.z; a[3] += q.w;
  }
  const int64_t base = (int64_t)co * Cg * KH * KW;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int r = r0 + i;
    int ci, kh, kw;
    if (mode == 2) {
      const int tap = r / 48, q = r - tap * 48;
      ci = q >> 4; kh = (tap / 3) * 4 + ((q >> 2) & 3); kw = (tap % 3) * 4 + (q & 3);
      if (kh >= KH || kw >= KW) continue;
    } else {
      const int tp = r / Cg;
      ci = r - tp * Cg; kh = tp / KW; kw = tp - kh * KW;
    }
    const int64_t e = base + (ci * KH + kh) * KW + kw;
    gw[e] = a[i];
    if (w) {
      float ww = w[e], vv = v[e];
      sgd_elem(ww, vv, a[i], mom, wdlr, lr);
      w[e] = ww;
      v[e] = vv;
      wb[e] = Num<T>::store(ww);
    }
  }
}

static dim3 wgrad_reduce_grid(int64_t outputs4) { return dim3((unsigned)((outputs4 + WR_Q - 1) / WR_Q)); }
static const SgdTarget kNoSgd{nullptr, nullptr, nullptr, {0.f, 0.f, 0.f}};

template <typename T>
static hipError_t conv_wgrad_t(const ConvShape& s, const void* dy, const void* x, float* part,
                               size_t part_bytes, float* gw, const SgdTarget& u, hipStream_t st,
                               const KTimer* kt) {
  constexpr int BM = 128, BN = 128;
  const int Cig = s.Cin / s.groups, Cog = s.Cout / s.groups;
  const int N = s.K * s.K * Cig, P = s.Nimg * s.Ho * s.Wo;
  const int tiles = cdiv(Cog, BM) * cdiv(N, BN) * s.groups;
  const int S = wgrad_splits(tiles, P);
  if ((size_t)s.groups * S * Cog * N * sizeof(float) > part_bytes) return hipErrorInvalidValue;
  const ConvGeom cg{s.H, s.W, s.Cin, Cig, s.K, s.K, s.stride, s.pad, s.Ho, s.Wo};
  EpF32 e;
  e.out = part; e.ldo = N; e.M = Cog; e.N = N; e.splits = S;
  hipError_t err;
  if (std::is_same<T, bf16>::value && s.Nimg % BK == 0) {
    DmaKOPix<BM> a;
    a.p = (const bf16*)dy; a.ld = s.Cout; a.rows = Cog; a.Nimg = s.Nimg; a.HoWo = s.Ho * s.Wo; a.Wo = s.Wo;
    a.gstride = Cog;
    DmaWgradBPix<BN> b;
    b.p = (const bf16*)x; b.cg = cg; b.rows = N; b.Nimg = s.Nimg;
    err = run_gemm<bf16, BM, BN, 2, 2>(a, b, e, Cog, N, P, s.groups, S, st, kt);
  } else {
    ColsLd<T, BM> a;
    a.p = (const T*)dy; a.ld = s.Cout; a.rows = Cog; a.K = P; a.gstride = Cog;
    WgradBLd<T, BN> b;
    b.p = (const T*)x; b.cg = cg; b.rows = N; b.P = P;
    err = run_gemm<T, BM, BN, 2, 2>(a, b, e, Cog, N, P, s.groups, S, st, kt);
  }
  if (err != hipSuccess) return err;
  if (N % 4) return hipErrorInvalidValue;
  hipLaunchKernelGGL((k_wgrad_finish<T>), dim3(s.Cout), dim3(WF_TPB), N * sizeof(float), st, part, S, Cog, N, Cig,
                     s.K, s.K, gw, u.w, u.v, (T*)u.wb, u.hy.lr, u.hy.mom, u.hy.wdlr);
  return hipGetLastError();
}

hipError_t conv_wgrad(DType dt, const ConvShape& s, const void* dy, const void* x, float* part,
                      size_t part_bytes, float* gw, const SgdTarget* u, hipStream_t st, const KTimer* kt) {
  const SgdTarget& t = u ? *u : kNoSgd;
  return dt == BF16 ? conv_wgrad_t<bf16>(s, dy, x, part, part_bytes, gw, t, st, kt)
                    : conv_wgrad_t<float>(s, dy, x, part, part_bytes, gw, t, st, kt);
}

template <typename T>
static hipError_t conv1_wgrad_t(int Nimg, const void* dy, const void* xs, float* part, size_t part_bytes,
                                float* gw, const SgdTarget& u, hipStream_t st, const KTimer* kt) {
  constexpr int BM = 128, BN = 128;
  const int N = S2D_K, P = Nimg * 3025;
  const int S = wgrad_splits(cdiv(96, BM) * cdiv(N, BN), P);
  if ((size_t)S * 96 * N * sizeof(float) > part_bytes) return hipErrorInvalidValue;
  EpF32 e;
  e.out = part; e.ldo = N; e.M = 96; e.N = N; e.splits = S;
  hipError_t err;
  // Pixel order (image-major): layer 1's large images make the pixel-major
  // order scatter its reads.
  ColsLd<T, BM> a;
  a.p = (const T*)dy; a.ld = 96; a.rows = 96; a.K = P; a.gstride = 0;
  WgradBLd<T, BN> b;
  b.p = (const T*)xs; b.cg = conv1_geom(); b.rows = N; b.P = P;
  err = run_gemm<T, BM, BN, 2, 2>(a, b, e, 96, N, P, 1, S, st, kt);
  if (err != hipSuccess) return err;
  hipLaunchKernelGGL((k_wgrad_reduce<T>), wgrad_reduce_grid(96 * N / 4), dim3(TPB), 0, st, part, 1, S, 96, N, 3,
                     11, 11, 2, gw, u.w, u.v, (T*)u.wb, u.hy.lr, u.hy.mom, u.hy.wdlr);
  return hipGetLastError();
}

// ---- layer 1 weight gradient, bf16: direct, with dY and the block rows in LDS
// dW'[co][k] = sum over pixels p of dY[p][co] * X'(p)[k], k = tap*48 + ci the
// space-to-depth order.  As an implicit GEMM (M = 96, N = 432, K = all
// pixels) every split reloads its pixels' dY once per 128 columns of N and
// gathers X' once per tap.  Here one workgroup per CU stays resident with all
// of dW' in its accumulators (eight waves, two per SIMD, each 3 or 4 of the 27
// fragments of 16 k x 96 channels) and walks the same tiles as the forward kernel: 4 output rows x 55
// columns of one image.  A tile's dY rows (220 pixels, then 4 zero rows) and
// its 6 input block rows are copied contiguously into LDS with direct-to-LDS
// loads, into one of two buffers while the previous tile is multiplied from
// the other; the first tile is copied with direct-to-LDS loads, later ones
// through registers between the products (see below).  The pixels are the
// contraction, 32 at a time: both operands are read as MFMA fragments with the
// transposing LDS read (lane t reads 4 values of one row; the 16 lanes of a
// group cover 4 pixel rows), the block rows as the first operand so that a
// lane ends with 4 consecutive k of one channel.  Each workgroup then writes
// its partial dW' (fp32) and k_wgrad_reduce sums the partials in workgroup
// order.  Batches whose dY exceeds 31-bit offsets run as image slices, each
// with its own partials.
constexpr int W1_PXT = 224;                                       // dY rows per tile in LDS (220, then zeros)
constexpr int W1_DYE = W1_PXT * 96;                               // bf16 elements of the dY tile
constexpr int W1_DYL = W1_DYE * 2 / 1024;                         // its direct-to-LDS loads
constexpr int W1_PTL = (C1_PROWS * S2D_B * S2D_C * 2 + 1023) / 1024;   // block-row loads
constexpr int W1_NL = W1_DYL + W1_PTL;                            // loads per tile
constexpr int W1_WAVES = 8;                                       // two waves per SIMD
constexpr int W1_NLW = (W1_NL + W1_WAVES - 1) / W1_WAVES;         // per wave, at most
constexpr int W1_BUF = W1_NL * 512;                               // bf16 elements per buffer
constexpr int W1_KF = S2D_K / 16;                                 // 27 fragments of 16 k
constexpr int W1_KFW = (W1_KF + W1_WAVES - 1) / W1_WAVES;         // per wave, at most
constexpr int W1_CF = 96 / 16;                                    // 6 fragments of 16 channels
constexpr int W1_CH = W1_PXT / 32;                                // pixel chunks of 32 per tile
constexpr int W1_MAXIMG = (int)(((int64_t)1 << 31) / (3025 * 96 * 2));   // images per slice
static_assert(W1_DYE * 2 % 1024 == 0 && S2D_K % 16 == 0 && S2D_C % 16 == 0, "fragment shapes");
static_assert(W1_PXT >= C1_ROWS * 55 && W1_PXT % 32 == 0, "tile shapes");
static_assert(2 * W1_BUF * 2 <= 160 * 1024, "two buffers fit in LDS");

static int w1_grid(int Nimg) { return std::min(256, (Nimg * C1_TPI + 7) / 8 * 8); }

__global__ void __launch_bounds__(64 * W1_WAVES) __attribute__((amdgpu_waves_per_eu(2, 2)))
k_conv1_wgrad(const bf16* __restrict__ dy, const bf16* __restrict__ xs, float* __restrict__ part, int Nimg) {
  __shared__ __attribute__((aligned(16))) bf16 lds[2 * W1_BUF];   // per buffer: [dY tile][block rows]
  typedef short v4s __attribute__((ext_vector_type(4)));
  typedef short v8s __attribute__((ext_vector_type(8)));
  typedef __attribute__((address_space(3))) v4s lds_v4s;
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  // XCD x takes a contiguous run of the tile order (as in the forward kernel)
  const int tiles = Nimg * C1_TPI;
  const int x = blockIdx.x & 7, per_x = gridDim.x >> 3;
  const int tq = tiles >> 3, tr = tiles & 7;
  const int t_end = x * tq + min(x, tr) + tq + (x < tr ? 1 : 0);
  int t = x * tq + min(x, tr) + (blockIdx.x >> 3);

  const __amdgpu_buffer_rsrc_t rsy = buf_rsrc(dy, (uint32_t)((int64_t)Nimg * 3025 * 96 * 2));
  const __amdgpu_buffer_rsrc_t rsx = buf_rsrc(xs, (uint32_t)((int64_t)Nimg * S2D_ELEMS * 2));
  // a tile's dY bytes (its valid pixels only; the rest of the 224 rows load
  // as zeros) and its block rows (6 rows from its first; past the input they
  // load as zeros, past the image they hold the next image's rows, which meet
  // only zero dY rows)
  auto geo = [](int tile, uint32_t& dbase, uint32_t& dlim, uint32_t& pbase) {
    const int n = tile / C1_TPI, r0 = (tile - n * C1_TPI) * C1_ROWS;
    dbase = (uint32_t)(((int64_t)n * 3025 + r0 * 55) * 96 * 2);
    dlim = (uint32_t)(min(C1_ROWS, 55 - r0) * 55 * 96 * 2);
    pbase = (uint32_t)(((int64_t)n * S2D_B + r0) * S2D_B * S2D_C * 2);
  };
  // The dY tile sits in LDS as two halves of 48 channels, [224 pixels][48]
  // (96-byte rows); LDS granule G of it holds granule dy_src(G) of the tile's
  // rows in memory (12 per pixel), at a byte offset that stays below dlim
  // exactly for the tile's valid pixels.
  auto dy_src = [](int G) {
    const int hh = G / (W1_PXT * 6), r = G - hh * (W1_PXT * 6), px = r / 6;
    return (uint32_t)((px * 12 + hh * 6 + (r - px * 6)) * 16);
  };
  // load i of this wave, j = wave + W1_WAVES i: 1 KB at granule 64 j of the buffer
  auto load = [&](int i, uint32_t dbase, uint32_t dlim, uint32_t pbase, bf16* buf) {
    const int j = wave + W1_WAVES * i;
    if (j < W1_DYL) {
      const uint32_t o = dy_src(j * 64 + lane);
      dma16(rsy, o < dlim ? dbase + o : BUF_OOB, buf + j * 512);
    } else if (j < W1_NL) {
      dma16(rsx, pbase + (uint32_t)((j - W1_DYL) * 1024 + lane * 16), buf + j * 512);
    }
  };
  if (t < t_end) {
    uint32_t dbase, dlim, pbase;
    geo(t, dbase, dlim, pbase);
#pragma unroll
    for (int i = 0; i < W1_NLW; ++i) load(i, dbase, dlim, pbase, lds);
  }
  // Later tiles come in through registers: load i of this wave fetches 16
  // bytes per lane and writes them to the same place in LDS as the
  // direct-to-LDS copy would, two chunks later.  (The compiler would make every
  // transposing LDS read wait for all direct-to-LDS loads issued before it, as
  // it cannot tell the buffers apart, and a chunk's reads follow the loads.)
  // No branches around these loads, so that the compiler can count them and
  // wait for each one alone: a wave short of a load repeats the previous
  // wave's last one (the same bytes to the same place), and after the last
  // tile the loads still run (zeros and rows of the first image, into the
  // buffer nothing reads again).
  typedef unsigned v4u __attribute__((ext_vector_type(4)));
  auto slot_of = [&](int i) { return min(wave + W1_WAVES * i, W1_NL - 1); };
  auto fetch = [&](int i, uint32_t dbase, uint32_t dlim, uint32_t pbase) {
    const int j = slot_of(i);
    const bool in_dy = j < W1_DYL;
    const uint32_t od = dy_src(min(j, W1_DYL - 1) * 64 + lane), op = (uint32_t)((j - W1_DYL) * 1024 + lane * 16);
    const uint32_t off = in_dy ? (od < dlim ? dbase + od : BUF_OOB) : pbase + op;
    return __builtin_amdgcn_raw_buffer_load_b128(in_dy ? rsy : rsx, off, 0, 0);
  };

  // Transposing-read addresses (elements within a buffer).  The MFMA's k
  // index kappa of a chunk (lane group g holds kappa = 8 g .. 8 g + 7) stands
  // for pixel 32 c + 16 h + 4 g + j, kappa = 8 g + 4 h + j: the same
  // order for both operands, so that each read of the 64 lanes covers 16
  // consecutive pixel rows, which at 96 bytes per row touch every bank once.
  // Lane (g, q) of chunk c, half h reads pixel row 32 c + 16 h + 4 g + q / 4
  // at 4 (q % 4) past the fragment's first column.
  const int g = lane >> 4, q = lane & 15;
  int dyo[W1_CH][2], pso[W1_CH][2];
#pragma unroll
  for (int c = 0; c < W1_CH; ++c)
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const int px = 32 * c + 16 * h + 4 * g + (q >> 2);
      const int lr = px / 55, col = px - lr * 55;
      dyo[c][h] = px * 48 + 4 * (q & 3);
      pso[c][h] = W1_DYE + (lr * S2D_B + col) * S2D_C + 4 * (q & 3);
    }
  // k-fragment i of this wave: kf = wave + W1_WAVES i, tap kf / 3, channels (kf % 3) * 16 ..
  int ko[W1_KFW];
#pragma unroll
  for (int i = 0; i < W1_KFW; ++i) {
    const int kf = min(wave + W1_WAVES * i, W1_KF - 1), tap = kf / 3, kh = tap / 3, kw = tap - kh * 3;
    ko[i] = (kh * S2D_B + kw) * S2D_C + (kf - tap * 3) * 16;
  }
  auto trd = [](const bf16* p, int o0, int o1) {
    const v4s lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4s*)(p + o0));
    const v4s hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4s*)(p + o1));
    return __builtin_bit_cast(bf16x8_t, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
  };
  const bool full = wave + W1_WAVES * (W1_KFW - 1) < W1_KF;   // this wave's last k-fragment exists

  f32x4_t acc[W1_KFW][W1_CF];
#pragma unroll
  for (int i = 0; i < W1_KFW; ++i)
#pragma unroll
    for (int j = 0; j < W1_CF; ++j) acc[i][j] = f32x4_t{0.f, 0.f, 0.f, 0.f};

  for (int it = 0; t < t_end; ++it) {
    const bf16* cur = lds + (it & 1) * W1_BUF;
    bf16* nxt = lds + ((it + 1) & 1) * W1_BUF;
    wait_vmcnt<0>();
    lds_barrier();   // tile t is in; every wave is done with the other buffer
    const int tn = t + per_x;
    const bool more = tn < t_end;
    uint32_t dbase = 0, dlim = 0, pbase = 0;
    if (more) geo(tn, dbase, dlim, pbase);

    bf16x8_t fa[2][W1_KFW], fb[2][W1_CF];
    // fragment f of a chunk: f < W1_CF the dY fragments (every product of the
    // chunk needs them), then the k-fragments in the order of use
    auto read_frag = [&](int c, int b, int f) {
      if (f < W1_CF) {
        const int ho = (f / 3) * (W1_PXT * 48) + (f % 3) * 16;   // channel half, column in it
        fb[b][f] = trd(cur, dyo[c][0] + ho, dyo[c][1] + ho);
      } else {
        const int i = f - W1_CF;
        if (i < W1_KFW - 1 || full) fa[b][i] = trd(cur, pso[c][0] + ko[i], pso[c][1] + ko[i]);
      }
    };
#pragma unroll
    for (int f = 0; f < W1_CF + W1_KFW; ++f) read_frag(0, 0, f);
    // The next chunk's fragments are read between this chunk's products, a
    // few per group of products: at most 15 LDS reads may be in flight, so a
    // chunk's 20 reads issued at once would stall the products behind them.
    // The next tile's data: LPC loads per chunk from chunk 0, each written to
    // LDS two chunks after it was issued.
    constexpr int FPG = (W1_CF + W1_KFW + W1_KFW - 1) / W1_KFW;   // fragments read per group
    constexpr int LPC = (W1_NLW + W1_CH - 3) / (W1_CH - 2);
    static_assert(LPC <= W1_KFW, "loads per group");
    v4u stage[3][LPC];
#pragma unroll
    for (int c = 0; c < W1_CH; ++c) {
#pragma unroll
      for (int i = 0; i < W1_KFW; ++i) {
        if (i < W1_KFW - 1 || full) {
#pragma unroll
          for (int j = 0; j < W1_CF; ++j)
            acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(fa[c & 1][i], fb[c & 1][j], acc[i][j], 0, 0, 0);
        }
        if (c + 1 < W1_CH) {
#pragma unroll
          for (int f = FPG * i; f < FPG * i + FPG; ++f)
            if (f < W1_CF + W1_KFW) read_frag(c + 1, (c + 1) & 1, f);
        }
        if (i < LPC) {
          const int lw = (c - 2) * LPC + i;   // written in this group: load issued two chunks ago
          if (c >= 2 && lw < W1_NLW) *reinterpret_cast<v4u*>(nxt + slot_of(lw) * 512 + lane * 8) = stage[(c - 2) % 3][i];
          const int li = c * LPC + i;         // issued in this group
          if (li < W1_NLW) stage[c % 3][i] = fetch(li, dbase, dlim, pbase);
        }
        __builtin_amdgcn_sched_barrier(0);
      }
    }
    t = tn;
  }

  // partial dW' of this workgroup: lane (g, q) holds k = 16 kf + 4 g .. + 3 of channel 16 j + q
  float* pw = part + (int64_t)blockIdx.x * 96 * S2D_K;
#pragma unroll
  for (int i = 0; i < W1_KFW; ++i) {
    if (i < W1_KFW - 1 || full) {
      const int kf = wave + W1_WAVES * i;
#pragma unroll
      for (int j = 0; j < W1_CF; ++j)
        *reinterpret_cast<f32x4_t*>(pw + (j * 16 + q) * S2D_K + kf * 16 + g * 4) = acc[i][j];
    }
  }
}

static int64_t conv1_wgrad_direct_splits(int Nimg) {
  int64_t s = 0;
  for (int n0 = 0; n0 < Nimg; n0 += W1_MAXIMG) s += w1_grid(std::min(W1_MAXIMG, Nimg - n0));
  return s;
}

static hipError_t conv1_wgrad_direct(int Nimg, const void* dy, const void* xs, float* part, size_t part_bytes,
                                     float* gw, const SgdTarget& u, hipStream_t st, const KTimer* kt) {
  const int64_t S = conv1_wgrad_direct_splits(Nimg);
  if (Nimg < 1 || (size_t)S * 96 * S2D_K * sizeof(float) > part_bytes) return hipErrorInvalidValue;
  rec_start(kt, st);
  float* pp = part;
  for (int n0 = 0; n0 < Nimg; n0 += W1_MAXIMG) {
    const int n = std::min(W1_MAXIMG, Nimg - n0);
    const int G = w1_grid(n);
    hipLaunchKernelGGL(k_conv1_wgrad, dim3(G), dim3(64 * W1_WAVES), 0, st, (const bf16*)dy + (int64_t)n0 * 3025 * 96,
                       (const bf16*)xs + (int64_t)n0 * S2D_ELEMS, pp, n);
    pp += (int64_t)G * 96 * S2D_K;
  }
  hipLaunchKernelGGL((k_wgrad_reduce<bf16>), wgrad_reduce_grid(96 * S2D_K / 4), dim3(TPB), 0, st, part, 1, (int)S,
                     96, S2D_K, 3, 11, 11, 2, gw, u.w, u.v, (bf16*)u.wb, u.hy.lr, u.hy.mom, u.hy.wdlr);
  rec_stop(kt, st);
  return hipGetLastError();
}

hipError_t conv1_wgrad(DType dt, int Nimg, const void* dy, const void* xs, float* part, size_t part_bytes,
                       float* gw, const SgdTarget* u, hipStream_t st, const KTimer* kt) {
  const SgdTarget& t = u ? *u : kNoSgd;
  return dt == BF16 ? conv1_wgrad_direct(Nimg, dy, xs, part, part_bytes, gw, t, st, kt)
                    : conv1_wgrad_t<float>(Nimg, dy, xs, part, part_bytes, gw, t, st, kt);
}

// ---- fully-connected layers
// FC layers at small batch stream their weights from HBM; split-K spreads
// that over the CUs in one round of at most one workgroup per CU, and bf16
// splits of 6 or more k-slices keep three slices in flight (four LDS stages,
// 128 KB) to cover the HBM latency.
static int fc_splits(int M, int N, int K) {
  const int tiles = cdiv(M, 128) * cdiv(N, 128);
  int want = 256 / tiles;
  if (want > 16) want = 16;
  // at full batch size, at least 8 k-slices per split: shorter splits spend
  // their time filling the pipeline and writing partials (FC8's data gradient,
  // 16 k-slices: 8 splits 17.4 us, 2 splits 15.7 us)
  const int kmax = cdiv(K, GEMM_BK) / 8;
  if (M >= 32 && want > kmax) want = kmax > 1 ? kmax : 1;
  return eff_splits(K, want);
}
template <typename T, class AL, class BL>
static hipError_t fc_gemm(const AL& a, const BL& b, const EpF32& e, int M, int N, int K, int S, hipStream_t st,
                          const KTimer* kt) {
  if constexpr (std::is_same<T, bf16>::value) {
    if (cdiv(cdiv(K, GEMM_BK), S) >= 6) return run_gemm<T, 128, 128, 2, 2, 4>(a, b, e, M, N, K, 1, S, st, kt);
  }
  return run_gemm<T, 128, 128, 2, 2, 2>(a, b, e, M, N, K, 1, S, st, kt);
}
size_t fc_fwd_part_bytes(int M, int K, int O) {
  return (size_t)fc_splits(M, O, K) * M * O * sizeof(float);
}

// Forward product of an FC layer for a handful of rows (M <= FC_ROWS_MAX,
// the batch-1 latency case), where MFMA tiles would be almost all padding
// and the run is one pass over the weight matrix.  One wave per output o
// walks row o of W in 8-element runs, lane l starting at 8 l and stepping
// 512, multiplies them with the same runs of every input row, and sums its
// lanes in a fixed order: part[m][o] = sum_k x[m][k] W[o][k] in fp32.
constexpr int FC_ROWS_MAX = 4;
template <typename T, int MR>
__global__ void __launch_bounds__(TPB) k_fc_rows(const T* __restrict__ x, const T* __restrict__ w, int K, int O,
                                                 float* __restrict__ part) {
  const int o = blockIdx.x * (TPB / 64) + (threadIdx.x >> 6), lane = threadIdx.x & 63;
  if (o >= O) return;   // whole waves; no barrier follows
  float acc[MR];
#pragma unroll
  for (int m = 0; m < MR; ++m) acc[m] = 0.f;
  const T* wr = w + (int64_t)o * K;
#pragma unroll 4
  for (int k = lane * 8; k < K; k += 512) {
    float wv[8];
    Pack8<T>::load(wr + k, wv);
#pragma unroll
    for (int m = 0; m < MR; ++m) {
      float xv[8];
      Pack8<T>::load(x + (int64_t)m * K + k, xv);
#pragma unroll
      for (int i = 0; i < 8; ++i) acc[m] = fmaf(xv[i], wv[i], acc[m]);
    }
  }
#pragma unroll
  for (int m = 0; m < MR; ++m) {
    float v = acc[m];
#pragma unroll
    for (int d = 32; d >= 1; d >>= 1) v += __shfl_xor(v, d);
    if (lane == 0) part[(int64_t)m * O + o] = v;
  }
}

// fp32 partial products part[s][m][o] of x W^T, S of them (set here): the
// MFMA GEMM split S ways over k, or k_fc_rows (S = 1) for a handful of rows.
template <typename T>
static hipError_t fc_partials(int M, int K, int O, const void* x, const void* w, float* part, size_t part_bytes,
                              hipStream_t st, const KTimer* kt, int& S) {
  if (M <= FC_ROWS_MAX && K % 8 == 0) {
    S = 1;
    if ((size_t)M * O * sizeof(float) > part_bytes) return hipErrorInvalidValue;
    const dim3 grid(cdiv(O, TPB / 64));
    const T* xp = (const T*)x;
    const T* wp = (const T*)w;
    rec_start(kt, st);
    switch (M) {
      case 1: hipLaunchKernelGGL((k_fc_rows<T, 1>), grid, dim3(TPB), 0, st, xp, wp, K, O, part); break;
      case 2: hipLaunchKernelGGL((k_fc_rows<T, 2>), grid, dim3(TPB), 0, st, xp, wp, K, O, part); break;
      case 3: hipLaunchKernelGGL((k_fc_rows<T, 3>), grid, dim3(TPB), 0, st, xp, wp, K, O, part); break;
      default: hipLaunchKernelGGL((k_fc_rows<T, 4>), grid, dim3(TPB), 0, st, xp, wp, K, O, part); break;
    }
    rec_stop(kt, st);
    return hipGetLastError();
  }
  S = fc_splits(M, O, K);
  if ((size_t)S * M * O * sizeof(float) > part_bytes) return hipErrorInvalidValue;
  RowsLd<T, 128> a;
  a.p = (const T*)x; a.ld = K; a.rows = M; a.K = K; a.gstride = 0;
  RowsLd<T, 128> bl;
  bl.p = (const T*)w; bl.ld = K; bl.rows = O; bl.K = K; bl.gstride = 0;
  EpF32 e;
  e.out = part; e.ldo = O; e.M = M; e.N = O; e.splits = S;
  return fc_gemm<T>(a, bl, e, M, O, K, S, st, kt);
}
size_t fc_dgrad_part_bytes(int M, int K, int O) {
  return (size_t)fc_splits(M, K, O) * M * K * sizeof(float);
}

// out[m * ldo + n] = epi(sum_s part[s][m][n] + b[n]) for 4 consecutive n per
// thread (ldo = N for the FC layers; mask, if any, has out's layout).
template <typename T>
__global__ void k_fc_reduce(const float* __restrict__ part, int S, int M, int N, int64_t ldo,
                            const T* __restrict__ bias, FcEpi ep, const T* __restrict__ mask, T* __restrict__ out,
                            float* __restrict__ out_f32) {
  const int64_t t = (int64_t)blockIdx.x * TPB + threadIdx.x;
  const int64_t total = (int64_t)M * N / 4;
  if (t >= total) return;
  const int64_t e0 = t * 4;
  const int m = (int)(e0 / N), n = (int)(e0 - (int64_t)m * N);
  float v[4] = {0.f, 0.f, 0.f, 0.f};
  // splits summed in order; eight partials in flight at a time instead of one
  // load's latency per split
  const float* pp = part + (int64_t)m * N + n;
  const int64_t sstride = (int64_t)M * N;
  int s = 0;
  for (; s + 8 <= S; s += 8) {
    float4 q[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) q[u] = *reinterpret_cast<const float4*>(pp + (s + u) * sstride);
#pragma unroll
    for (int u = 0; u < 8; ++u) { v[0] += q[u].x; v[1] += q[u].y; v[2] += q[u].z; v[3] += q[u].w; }
  }
  for (; s < S; ++s) {
    const float4 q = *reinterpret_cast<const float4*>(pp + s * sstride);
    v[0] += q.x; v[1] += q.y; v[2] += q.z; v[3] += q.w;
  }
  if (bias) {
#pragma unroll
    for (int i = 0; i < 4; ++i) v[i] += Num<T>::load(bias[n + i]);
  }
  if (ep.relu) {
#pragma unroll
    for (int i = 0; i < 4; ++i) v[i] = v[i] > 0.f ? v[i] : 0.f;
  }
  if (ep.drop == 1) {
    // element e = m*N + n (N % 4 == 0, so the four share one Philox block)
    const uint4 r = philox4x32_10(make_uint4((uint32_t)(e0 >> 2), (uint32_t)ep.layer, (uint32_t)ep.step,
                                             (uint32_t)(ep.step >> 32)),
                                  (uint32_t)ep.seed, (uint32_t)(ep.seed >> 32));
    const uint32_t w[4] = {r.x, r.y, r.z, r.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) v[i] = w[i] < ep.thresh ? 0.f : v[i];
  } else if (ep.drop == 2) {
#pragma unroll
    for (int i = 0; i < 4; ++i) v[i] *= ep.scale;
  }
  const int64_t o = (int64_t)m * ldo + n;
  if (mask) {
#pragma unroll
    for (int i = 0; i < 4; ++i) v[i] = Num<T>::load(mask[o + i]) > 0.f ? v[i] : 0.f;
  }
  if (out_f32) {
    *reinterpret_cast<float4*>(out_f32 + o) = make_float4(v[0], v[1], v[2], v[3]);
  } else {
#pragma unroll
    for (int i = 0; i < 4; ++i) out[o + i] = Num<T>::store(v[i]);
  }
}

template <typename T>
static hipError_t fc_fwd_t(int M, int K, int O, const void* x, const void* w, const void* b,
                           const FcEpi& ep, void* y, float* y_f32, float* part, size_t part_bytes,
                           hipStream_t st, const KTimer* kt) {
  int S = 1;
  hipError_t err = fc_partials<T>(M, K, O, x, w, part, part_bytes, st, kt, S);
  if (err != hipSuccess) return err;
  hipLaunchKernelGGL((k_fc_reduce<T>), grid1d((int64_t)M * O / 4), dim3(TPB), 0, st, part, S, M, O, (int64_t)O,
                     (const T*)b, ep, (const T*)nullptr, (T*)y, y_f32);
  return hipGetLastError();
}

hipError_t fc_fwd(DType dt, int M, int K, int O, const void* x, const void* w, const void* b,
                  const FcEpi& ep, void* y, float* y_f32, float* part, size_t part_bytes, hipStream_t st,
                  const KTimer* kt) {
  return dt == BF16 ? fc_fwd_t<bf16>(M, K, O, x, w, b, ep, y, y_f32, part, part_bytes, st, kt)
                    : fc_fwd_t<float>(M, K, O, x, w, b, ep, y, y_f32, part, part_bytes, st, kt);
}

template <typename T>
static hipError_t fc_dgrad_t(int M, int K, int O, const void* dy, const void* w, const void* mask,
                             void* dx, float* part, size_t part_bytes, hipStream_t st, const KTimer* kt) {
  constexpr int BM = 128, BN = 128;
  const int S = fc_splits(M, K, O);
  if ((size_t)S * M * K * sizeof(float) > part_bytes) return hipErrorInvalidValue;
  RowsLd<T, BM> a;
  a.p = (const T*)dy; a.ld = O; a.rows = M; a.K = O; a.gstride = 0;
  ColsLd<T, BN> bl;
  bl.p = (const T*)w; bl.ld = K; bl.rows = K; bl.K = O; bl.gstride = 0;
  EpF32 e;
  e.out = part; e.ldo = K; e.M = M; e.N = K; e.splits = S;
  hipError_t err = fc_gemm<T>(a, bl, e, M, K, O, S, st, kt);
  if (err != hipSuccess) return err;
  FcEpi none{};
  hipLaunchKernelGGL((k_fc_reduce<T>), grid1d((int64_t)M * K / 4), dim3(TPB), 0, st, part, S, M, K, (int64_t)K,
                     (const T*)nullptr, none, (const T*)mask, (T*)dx, (float*)nullptr);
  return hipGetLastError();
}

hipError_t fc_dgrad(DType dt, int M, int K, int O, const void* dy, const void* w, const void* mask,
                    void* dx, float* part, size_t part_bytes, hipStream_t st, const KTimer* kt) {
  return dt == BF16 ? fc_dgrad_t<bf16>(M, K, O, dy, w, mask, dx, part, part_bytes, st, kt)
                    : fc_dgrad_t<float>(M, K, O, dy, w, mask, dx, part, part_bytes, st, kt);
}

// Epilogue of the FC weight-gradient GEMM: the fp32 gradient of 8 weights
// w[m][n .. n+7] goes straight into the SGD update of master w, momentum v
// and working copy wb (sgd_elem, as every other tensor's update).
// w and v are fetched ahead (prefetch) while the accumulators are staged.
template <typename T>
struct EpSgd {
  static constexpr bool prefetches = true;
  struct State { float4 w0, w1, v0, v1; };
  float* w; float* v; T* wb; int ldo, M, N; SgdHyper h;
  __device__ __forceinline__ State prefetch(int m, int n) const {
    State st{};
    if (m < M && n < N) {
      const int64_t o = (int64_t)m * ldo + n;
      st.w0 = *reinterpret_cast<const float4*>(w + o);
      st.w1 = *reinterpret_cast<const float4*>(w + o + 4);
      st.v0 = *reinterpret_cast<const float4*>(v + o);
      st.v1 = *reinterpret_cast<const float4*>(v + o + 4);
    }
    return st;
  }
  __device__ __forceinline__ void apply(int m, int n, const float* g, const State& st) const {
    if (m >= M || n >= N) return;
    const int64_t o = (int64_t)m * ldo + n;
    float wv[8] = {st.w0.x, st.w0.y, st.w0.z, st.w0.w, st.w1.x, st.w1.y, st.w1.z, st.w1.w};
    float vv[8] = {st.v0.x, st.v0.y, st.v0.z, st.v0.w, st.v1.x, st.v1.y, st.v1.z, st.v1.w};
#pragma unroll
    for (int i = 0; i < 8; ++i) sgd_elem(wv[i], vv[i], g[i], h.mom, h.wdlr, h.lr);
    // Nothing reads these before the next step: non-temporal stores keep the
    // last-level cache clean for the streaming reads of the layers that follow.
    Pack8<float>::store_nt(w + o, wv);
    Pack8<float>::store_nt(v + o, vv);
    Pack8<T>::store_nt(wb + o, wv);
  }
  // per-chunk form (used when a tile's chunk count does not split evenly)
  __device__ __forceinline__ void operator()(int m, int n, int, int, const float* g) const {
    apply(m, n, g, prefetch(m, n));
  }
};

constexpr int FC_WGRAD_STRIP = 18;
template <typename T>
static hipError_t fc_wgrad_sgd_t(int M, int K, int O, const void* dy, const void* x, const SgdHyper& h,
                                 float* w, float* v, void* wb, hipStream_t st, const KTimer* kt) {
  constexpr int BM = 128, BN = 128;
  if (K % 8) return hipErrorInvalidValue;
  ColsLd<T, BM> a;
  a.p = (const T*)dy; a.ld = O; a.rows = O; a.K = M; a.gstride = 0;
  ColsLd<T, BN> bl;
  bl.p = (const T*)x; bl.ld = K; bl.rows = K; bl.K = M; bl.gstride = 0;
  EpSgd<T> e;
  e.w = w; e.v = v; e.wb = (T*)wb; e.ldo = K; e.M = O; e.N = K; e.h = h;
  return run_gemm<T, BM, BN, 2, 2>(a, bl, e, O, K, M, 1, 1, st, kt, FC_WGRAD_STRIP);
}

hipError_t fc_wgrad_sgd(DType dt, int M, int K, int O, const void* dy, const void* x, const SgdHyper& h,
                        float* w, float* v, void* wb, hipStream_t st, const KTimer* kt) {
  return dt == BF16 ? fc_wgrad_sgd_t<bf16>(M, K, O, dy, x, h, w, v, wb, st, kt)
                    : fc_wgrad_sgd_t<float>(M, K, O, dy, x, h, w, v, wb, st, kt);
}

// =========================================================================
// Weight re-layouts
// =========================================================================
// All in one launch.  Jobs:
//   W1S    layer 1 over 4x4 pixel blocks: W'[co][kh'][kw'][c*16+dh*4+dw] =
//          W[co][c][4kh'+dh][4kw'+dw], zero where 4kh'+dh or 4kw'+dw >= 11;
//          one output element per thread;
//   KHWC   forward rows [co], k = (tap, ci), or with `blocked`
//          k = (ci / 64, tap, ci % 64), tap = kh*K + kw: one workgroup per co
//          copies the co slice (Cg*K*K contiguous elements) into LDS and
//          writes it back permuted (the destination slice is contiguous too);
//   DGRAD  data-gradient rows [g][ci], k over (flipped tap, output channel col
//          of the group): k = (tap, col), or with `blocked`
//          k = (col / 64, tap, col % 64): a 64 x 64 tile transpose through LDS
//          of (64 output channels col) x (64 consecutive (ci, tap) entries).
// Reads and writes of neighbouring threads are contiguous in every job.
constexpr int WPREP_T = 64;                              // DGRAD tile edge
constexpr int WPREP_LDS_ELEMS = 4160;                    // >= max(Cg*K*K) = 3456 and 64 x 65
struct PrepArgs {
  const void* src[WPREP_MAX];
  void* dst[WPREP_MAX];
  int kind[WPREP_MAX], Cog[WPREP_MAX], Cig[WPREP_MAX], K[WPREP_MAX], blocked[WPREP_MAX], count[WPREP_MAX];
  int bstart[WPREP_MAX + 1];   // first block of each job
  int n;
};

template <typename T>
__device__ __forceinline__ void prep_block(int bid, const PrepArgs& a) {
  __shared__ __attribute__((aligned(16))) T tile[WPREP_LDS_ELEMS];
  const int tid = threadIdx.x;
  int j = 0;
#pragma unroll
  for (int q = 1; q < WPREP_MAX; ++q) j += (q < a.n && bid >= a.bstart[q]) ? 1 : 0;
  const int local = bid - a.bstart[j];
  const T* __restrict__ src = static_cast<const T*>(a.src[j]);
  T* __restrict__ dst = static_cast<T*>(a.dst[j]);
  const int kind = a.kind[j];
  if (kind == WPREP_W1S) {
    const int i = local * TPB + tid;
    if (i >= a.count[j]) return;
    const int co = i / S2D_K, r = i - co * S2D_K;
    const int tap = r / S2D_C, q = r - tap * S2D_C;
    const int kh = (tap / 3) * 4 + ((q >> 2) & 3), kw = (tap % 3) * 4 + (q & 3), c = q >> 4;
    dst[i] = (kh < 11 && kw < 11) ? src[((co * 3 + c) * 11 + kh) * 11 + kw] : T(0);
    return;
  }
  const int KK = a.K[j] * a.K[j], blocked = a.blocked[j];
  constexpr int V = 16 / (int)sizeof(T);   // elements per 16-byte access
  if (kind == WPREP_KHWC) {
    // n = Cg*K*K is a multiple of V (host-checked): 16-byte copies in and out
    const int Cg = a.Cig[j], n = Cg * KK, co = local;
    const T* s = src + (int64_t)co * n;
    for (int e = tid * V; e < n; e += TPB * V) *reinterpret_cast<uint4*>(tile + e) = *reinterpret_cast<const uint4*>(s + e);
    __syncthreads();
    T* d = dst + (int64_t)co * n;
    for (int o0 = tid * V; o0 < n; o0 += TPB * V) {
      T v[V];
#pragma unroll
      for (int q = 0; q < V; ++q) {
        const int o = o0 + q;
        int ci, tap;
        if (blocked) {
          const int t2 = o / GEMM_BK;
          tap = t2 % KK;
          ci = (t2 / KK) * GEMM_BK + (o - t2 * GEMM_BK);
        } else {
          tap = o / Cg;
          ci = o - tap * Cg;
        }
        v[q] = tile[ci * KK + tap];
      }
      *reinterpret_cast<uint4*>(d + o0) = pack_u4(v);
    }
    return;
  }
  // DGRAD: tile (g, col block, e block), e = ci*KK + tap over W[g*Cog + col][ci][tap];
  // Cog and Cig*KK are multiples of V (host-checked), so every 16-byte access is whole
  const int Cog = a.Cog[j], Cig = a.Cig[j], nE = Cig * KK;
  const int ncb = (Cog + WPREP_T - 1) / WPREP_T, neb = (nE + WPREP_T - 1) / WPREP_T;
  const int g = local / (ncb * neb), rem = local - g * ncb * neb;
  const int col0 = (rem / neb) * WPREP_T, e0 = (rem % neb) * WPREP_T;
  constexpr int VPR = WPREP_T / V;   // 16-byte pieces per tile row
  for (int idx = tid; idx < WPREP_T * VPR; idx += TPB) {
    const int c = idx / VPR, e = (idx - c * VPR) * V;
    if (col0 + c < Cog && e0 + e < nE) {
      T v[V];
      unpack_u4(*reinterpret_cast<const uint4*>(src + (int64_t)(g * Cog + col0 + c) * nE + e0 + e), v);
#pragma unroll
      for (int q = 0; q < V; ++q) tile[c * (WPREP_T + 1) + e + q] = v[q];
    }
  }
  __syncthreads();
  const int nblk = Cog / GEMM_BK;
  for (int idx = tid; idx < WPREP_T * VPR; idx += TPB) {
    const int e = idx / VPR, c = (idx - e * VPR) * V;
    const int col = col0 + c, ee = e0 + e;
    if (col >= Cog || ee >= nE) continue;
    const int ci = ee / KK, tapo = KK - 1 - (ee - ci * KK);   // output tap takes the flipped source tap
    T v[V];
#pragma unroll
    for (int q = 0; q < V; ++q) v[q] = tile[(c + q) * (WPREP_T + 1) + e];
    int64_t o;
    if (blocked) o = (((int64_t)(g * Cig + ci) * nblk + col / GEMM_BK) * KK + tapo) * GEMM_BK + (col % GEMM_BK);
    else o = ((int64_t)(g * Cig + ci) * KK + tapo) * Cog + col;
    *reinterpret_cast<uint4*>(dst + o) = pack_u4(v);
  }
}

bool im2col_blocked(DType dt, int Cg) { return dt == BF16 && Cg % GEMM_BK == 0; }

// Start of every call, one launch: the weight re-layouts (workgroups below
// a.bstart[a.n]) and the layer-1 input staging (one workgroup per image and
// block row after them) are independent of each other.
template <typename T>
__global__ void __launch_bounds__(TPB) k_stage(PrepArgs a, const T* __restrict__ x, T* __restrict__ xs, int Hs,
                                               int Ws, int kind, AugSrc aug, int64_t total) {
  const int prep_blocks = a.bstart[a.n];
  if ((int)blockIdx.x < prep_blocks) prep_block<T>(blockIdx.x, a);
  else s2d_block<T>(blockIdx.x - prep_blocks, x, xs, Hs, Ws, kind, aug, total);
}

hipError_t stage_inputs(DType dt, const WeightPrep* jobs, int n, const void* x, int Hs, int Ws, int kind,
                        const AugSrc* aug, int Nimg, void* xs, hipStream_t st, const KTimer* kt) {
  if (n < 1 || n > WPREP_MAX) return hipErrorInvalidValue;
  if (kind != SRC_IMAGES && kind != SRC_TENVIEW && kind != SRC_AUGMENT) return hipErrorInvalidValue;
  if (kind == SRC_AUGMENT && (!aug || Hs < 227 || Ws < 227)) return hipErrorInvalidValue;
  const AugSrc ag = kind == SRC_AUGMENT ? *aug : AugSrc{nullptr, nullptr, nullptr, nullptr};
  PrepArgs a = {};
  a.n = n;
  int blocks = 0;
  for (int j = 0; j < n; ++j) {
    const WeightPrep& w = jobs[j];
    int64_t count;
    a.src[j] = w.src;
    a.dst[j] = w.dst;
    a.kind[j] = w.kind;
    a.K[j] = w.K;
    switch (w.kind) {
      case WPREP_W1S:
        count = (int64_t)S2D_W_ELEMS;
        break;
      case WPREP_KHWC:   // Cig = input channels per group; one workgroup per co
        if (w.Cig * w.K * w.K > WPREP_LDS_ELEMS || (w.Cig * w.K * w.K) % 8) return hipErrorInvalidValue;
        a.Cig[j] = w.Cig;
        a.blocked[j] = im2col_blocked(dt, w.Cig) ? 1 : 0;
        count = w.Cout;
        break;
      case WPREP_DGRAD:  // one workgroup per 64 x 64 tile
        if (w.G < 1 || w.Cout % w.G || (w.Cout / w.G) % 8 || (w.Cig * w.K * w.K) % 8) return hipErrorInvalidValue;
        a.Cog[j] = w.Cout / w.G;
        a.Cig[j] = w.Cig;
        a.blocked[j] = im2col_blocked(dt, a.Cog[j]) ? 1 : 0;
        count = (int64_t)w.G * cdiv(a.Cog[j], WPREP_T) * cdiv((int64_t)w.Cig * w.K * w.K, WPREP_T);
        break;
      default:
        return hipErrorInvalidValue;
    }
    if (count > (int64_t)1 << 30) return hipErrorInvalidValue;
    a.count[j] = (int)count;   // W1S: elements; KHWC, DGRAD: workgroups
    a.bstart[j] = blocks;
    blocks += w.kind == WPREP_W1S ? cdiv(count, TPB) : (int)count;
  }
  a.bstart[n] = blocks;
  const int64_t total = (int64_t)(kind == SRC_TENVIEW ? Nimg / 10 : Nimg) * 3 * Hs * Ws;
  const dim3 g(blocks + Nimg * S2D_B);
  rec_start(kt, st);
  if (dt == BF16)
    hipLaunchKernelGGL((k_stage<bf16>), g, dim3(TPB), 0, st, a, (const bf16*)x, (bf16*)xs, Hs, Ws, kind, ag,
                       total);
  else
    hipLaunchKernelGGL((k_stage<float>), g, dim3(TPB), 0, st, a, (const float*)x, (float*)xs, Hs, Ws, kind, ag,
                       total);
  rec_stop(kt, st);
  return hipGetLastError();
}

// The augmented patches as NCHW images, one thread per output element (the
// same per-element arithmetic as the staging above).
template <typename T>
__global__ void __launch_bounds__(TPB) k_augment(const T* __restrict__ src, int Hs, int Ws, AugSrc aug,
                                                 int64_t total, T* __restrict__ out) {
  const int64_t e = (int64_t)blockIdx.x * TPB + threadIdx.x;
  if (e >= total) return;
  constexpr int P = 227 * 227;
  const int n = (int)(e / (3 * P));
  const int rem = (int)(e - (int64_t)n * 3 * P);
  const int c = rem / P, yx = rem - c * P, y = yx / 227, xo = yx - y * 227;
  int y0, x0, flip;
  aug_patch(aug, n, Hs, Ws, y0, x0, flip);
  const int xi = x0 + (flip ? 226 - xo : xo);
  const T v = src[(((int64_t)n * 3 + c) * Hs + y0 + y) * Ws + xi];
  out[e] = aug_value(v, aug_shift(aug, n, c));
}

hipError_t augment_images(DType dt, const void* src, int Hs, int Ws, const AugSrc& aug, int Nimg, void* x_out,
                          hipStream_t st) {
  if (Hs < 227 || Ws < 227 || Nimg < 0) return hipErrorInvalidValue;
  const int64_t total = (int64_t)Nimg * 3 * 227 * 227;
  if (total == 0) return hipSuccess;
  if (dt == BF16)
    hipLaunchKernelGGL((k_augment<bf16>), grid1d(total), dim3(TPB), 0, st, (const bf16*)src, Hs, Ws, aug, total,
                       (bf16*)x_out);
  else
    hipLaunchKernelGGL((k_augment<float>), grid1d(total), dim3(TPB), 0, st, (const float*)src, Hs, Ws, aug, total,
                       (float*)x_out);
  return hipGetLastError();
}

// ---- principal components of the RGB values (section 4.1: the 3 x 3
// covariance of the RGB values of all pixels, its eigenvectors and
// eigenvalues).  Pass 1: PCA_BLOCKS workgroups each accumulate, in fp64, the
// nine moments sum r, g, b and sum rr, rg, rb, gg, gb, bb over a grid-stride
// range of pixels, reduced in the workgroup in a fixed tree order.  (For bf16
// inputs every product and partial sum is exact in fp64.)  Pass 2: one
// workgroup sums the partials in a fixed order, forms the covariance
// (E[x x^T] - mean mean^T; the fp64 moments keep the cancellation harmless
// unless the mean exceeds the spread by ~10^4) and diagonalises it.
constexpr int PCA_BLOCKS = 256;
size_t rgb_pca_scratch_bytes() { return (size_t)PCA_BLOCKS * 9 * sizeof(double); }

// in-place fixed-order tree sum of v[0..TPB) in LDS; result in v[0]
__device__ __forceinline__ void tree_sum(double* v) {
  for (int w = TPB / 2; w > 0; w >>= 1) {
    if ((int)threadIdx.x < w) v[threadIdx.x] += v[threadIdx.x + w];
    __syncthreads();
  }
}

__device__ __forceinline__ void rgb_accumulate(double (&m)[9], double r, double g, double bl) {
  m[0] += r; m[1] += g; m[2] += bl;
  m[3] += r * r; m[4] += r * g; m[5] += r * bl;
  m[6] += g * g; m[7] += g * bl; m[8] += bl * bl;
}

// Planes whose size is a multiple of 8 are read as runs of 8 pixels (one
// 16-byte load per channel for bf16) so that many loads are in flight; other
// sizes pixel by pixel.
template <typename T>
__global__ void __launch_bounds__(TPB) k_rgb_moments(const T* __restrict__ src, int64_t HW, int64_t P,
                                                     double* __restrict__ part) {
  __shared__ double red[9][TPB];
  double m[9] = {0., 0., 0., 0., 0., 0., 0., 0., 0.};
  const int64_t stride = (int64_t)gridDim.x * TPB;
  if (HW % 8 == 0) {
    const int64_t runs = P / 8;
#pragma unroll 2
    for (int64_t c = (int64_t)blockIdx.x * TPB + threadIdx.x; c < runs; c += stride) {
      const int64_t p = c * 8, img = p / HW, q = p - img * HW;
      const T* b = src + img * 3 * HW + q;
      float r[8], g[8], bl[8];
      Pack8<T>::load(b, r);
      Pack8<T>::load(b + HW, g);
      Pack8<T>::load(b + 2 * HW, bl);
#pragma unroll
      for (int i = 0; i < 8; ++i) rgb_accumulate(m, r[i], g[i], bl[i]);
    }
  } else {
    for (int64_t p = (int64_t)blockIdx.x * TPB + threadIdx.x; p < P; p += stride) {
      const int64_t img = p / HW, q = p - img * HW;
      const T* b = src + img * 3 * HW + q;
      rgb_accumulate(m, Num<T>::load(b[0]), Num<T>::load(b[HW]), Num<T>::load(b[2 * HW]));
    }
  }
#pragma unroll
  for (int k = 0; k < 9; ++k) red[k][threadIdx.x] = m[k];
  __syncthreads();
  for (int w = TPB / 2; w > 0; w >>= 1) {
    if ((int)threadIdx.x < w) {
#pragma unroll
      for (int k = 0; k < 9; ++k) red[k][threadIdx.x] += red[k][threadIdx.x + w];
    }
    __syncthreads();
  }
  if (threadIdx.x < 9) part[blockIdx.x * 9 + threadIdx.x] = red[threadIdx.x][0];
}

// Cyclic Jacobi eigenvalue iteration on a symmetric 3 x 3 matrix a (row
// major): each rotation in the (p, q) plane, with t = tan(phi) the smaller
// root of t^2 + 2 theta t - 1 = 0, theta = (a_qq - a_pp) / (2 a_pq), zeroes
// a_pq; the rotations accumulate in v.  Sweeps stop when the off-diagonal
// mass is negligible against the diagonal (at most 50 sweeps).
__device__ void jacobi3(double a[3][3], double v[3][3]) {
  for (int i = 0; i < 3; ++i)
    for (int j = 0; j < 3; ++j) v[i][j] = i == j ? 1. : 0.;
  const int P[3] = {0, 0, 1}, Q[3] = {1, 2, 2};
  for (int sweep = 0; sweep < 50; ++sweep) {
    const double off = a[0][1] * a[0][1] + a[0][2] * a[0][2] + a[1][2] * a[1][2];
    const double dia = a[0][0] * a[0][0] + a[1][1] * a[1][1] + a[2][2] * a[2][2];
    if (off <= 1e-34 * dia || off == 0.) break;
    for (int k = 0; k < 3; ++k) {
      const int p = P[k], q = Q[k];
      const double apq = a[p][q];
      if (apq == 0.) continue;
      const double theta = (a[q][q] - a[p][p]) / (2. * apq);
      double t = 1. / (fabs(theta) + sqrt(theta * theta + 1.));
      if (fabs(theta) > 1e150) t = 0.5 / fabs(theta);
      if (theta < 0.) t = -t;
      const double c = 1. / sqrt(t * t + 1.), s = t * c;
      a[p][p] -= t * apq;
      a[q][q] += t * apq;
      a[p][q] = a[q][p] = 0.;
      const int r = 3 - p - q;   // the remaining index
      const double arp = a[r][p], arq = a[r][q];
      a[r][p] = a[p][r] = c * arp - s * arq;
      a[r][q] = a[q][r] = s * arp + c * arq;
      for (int i = 0; i < 3; ++i) {
        const double vip = v[i][p], viq = v[i][q];
        v[i][p] = c * vip - s * viq;
        v[i][q] = s * vip + c * viq;
      }
    }
  }
}

__global__ void __launch_bounds__(TPB) k_rgb_pca_finish(const double* __restrict__ part, int nblk, int64_t P,
                                                        float* __restrict__ eigval, float* __restrict__ eigvec) {
  __shared__ double red[TPB];
  __shared__ double mom[9];
  for (int k = 0; k < 9; ++k) {
    double acc = 0.;   // partials t, t + TPB, ... in order, then the tree
    for (int b = threadIdx.x; b < nblk; b += TPB) acc += part[b * 9 + k];
    red[threadIdx.x] = acc;
    __syncthreads();
    tree_sum(red);
    if (threadIdx.x == 0) mom[k] = red[0];
    __syncthreads();
  }
  if (threadIdx.x != 0) return;
  const double inv = 1. / (double)P;
  const double mean[3] = {mom[0] * inv, mom[1] * inv, mom[2] * inv};
  const int idx[3][3] = {{3, 4, 5}, {4, 6, 7}, {5, 7, 8}};
  double a[3][3], v[3][3];
  for (int i = 0; i < 3; ++i)
    for (int j = 0; j < 3; ++j) a[i][j] = mom[idx[i][j]] * inv - mean[i] * mean[j];
  jacobi3(a, v);
  // eigenvalues in descending order, ties keep the lower index first
  int ord[3] = {0, 1, 2};
  for (int i = 0; i < 2; ++i)
    for (int j = 0; j < 2 - i; ++j)
      if (a[ord[j + 1]][ord[j + 1]] > a[ord[j]][ord[j]]) { const int t = ord[j]; ord[j] = ord[j + 1]; ord[j + 1] = t; }
  for (int i = 0; i < 3; ++i) {
    const int k = ord[i];
    int big = 0;
    for (int r = 1; r < 3; ++r)
      if (fabs(v[r][k]) > fabs(v[big][k])) big = r;
    const double sg = v[big][k] < 0. ? -1. : 1.;
    eigval[i] = (float)a[k][k];
    for (int r = 0; r < 3; ++r) eigvec[3 * r + i] = (float)(sg * v[r][k]);
  }
}

hipError_t rgb_pca(DType dt, const void* src, int n, int H, int W, float* eigval, float* eigvec, void* scratch,
                   hipStream_t st, const KTimer* kt) {
  if (n < 1 || H < 1 || W < 1) return hipErrorInvalidValue;
  const int64_t HW = (int64_t)H * W, P = (int64_t)n * HW;
  double* part = (double*)scratch;
  rec_start(kt, st);
  if (dt == BF16)
    hipLaunchKernelGGL((k_rgb_moments<bf16>), dim3(PCA_BLOCKS), dim3(TPB), 0, st, (const bf16*)src, HW, P, part);
  else
    hipLaunchKernelGGL((k_rgb_moments<float>), dim3(PCA_BLOCKS), dim3(TPB), 0, st, (const float*)src, HW, P, part);
  hipLaunchKernelGGL(k_rgb_pca_finish, dim3(1), dim3(TPB), 0, st, (const double*)part, PCA_BLOCKS, P, eigval,
                     eigvec);
  rec_stop(kt, st);
  return hipGetLastError();
}

// =========================================================================
// Local response normalisation across channels, NHWC
//   b_i = a_i * S_i^-beta,  S_i = k + alpha * sum_{|j-i| <= half, 0 <= j < C} a_j^2
// =========================================================================
// Loads channels c0-8 .. c0+15 of one pixel (zero outside [0, C)).
template <typename T>
__device__ __forceinline__ void load24(const T* px, int c0, int C, float* v) {
#pragma unroll
  for (int q = 0; q < 3; ++q) {
    const int cc = c0 + (q - 1) * 8;
    if (cc >= 0 && cc < C) Pack8<T>::load(px + cc, v + q * 8);
    else {
#pragma unroll
      for (int i = 0; i < 8; ++i) v[q * 8 + i] = 0.f;
    }
  }
}

// LRN kernels take the window half-width H and the beta == 3/4 case as
// compile-time parameters, so every loop below unrolls completely.
// S = k + alpha * sum >= k > 0 is a normal number, so the hardware reciprocal
// square root and square root (about 1 ulp each) need no range scaling:
// with beta == 3/4, r = rsq(S), S^-beta = r sqrt(r), S^(-beta-1) = S^-beta r^2.
template <bool B075>
__device__ __forceinline__ void lrn_pows(float S, float beta, float& p, float& q) {
  if (B075) {
    const float r = __builtin_amdgcn_rsqf(S);
    p = r * __builtin_amdgcn_sqrtf(r);
    q = p * r * r;
  } else {
    p = exp2f(-beta * log2f(S));
    q = p / S;
  }
}

// LRN of 8 channels c0 .. c0+7 of one pixel; v holds channels c0-8 .. c0+15.
template <int H, bool B075>
__device__ __forceinline__ void lrn8(const float* v, float k, float alpha, float beta, float* o) {
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    float s = 0.f;
#pragma unroll
    for (int j = -H; j <= H; ++j) s += v[8 + i + j] * v[8 + i + j];
    float p, q;
    lrn_pows<B075>(k + alpha * s, beta, p, q);
    o[i] = v[8 + i] * p;
  }
}

// Backward of LRN fused with the preceding ReLU's mask [a > 0], for channels
// c0 .. c0+7 of one pixel:
//   da_j = g_j S_j^-beta - 2 alpha beta a_j sum_{|i-j| <= H} g_i a_i S_i^(-beta-1)
// av holds a over c0-8 .. c0+15 and gv holds g over the same channels (only
// c0-H .. c0+7+H of g and c0-2H .. c0+7+2H of a are used; H <= 4).
template <int H, bool B075>
__device__ __forceinline__ void lrn_bwd8(const float* av, const float* gv, float k, float alpha, float beta,
                                         float* o) {
  constexpr int NR = 8 + 2 * H;
  float pb[NR], tt[NR];
#pragma unroll
  for (int r = 0; r < NR; ++r) {
    const int rel = 8 - H + r;
    float s = 0.f;
#pragma unroll
    for (int j = -H; j <= H; ++j) s += av[rel + j] * av[rel + j];
    float p, q;
    lrn_pows<B075>(k + alpha * s, beta, p, q);
    pb[r] = p;
    tt[r] = gv[rel] * av[rel] * q;
  }
  const float c2 = 2.f * alpha * beta;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    float cross = 0.f;
#pragma unroll
    for (int j = -H; j <= H; ++j) cross += tt[i + H + j];
    const float aj = av[8 + i];
    const float d = gv[8 + i] * pb[i + H] - c2 * aj * cross;
    o[i] = aj > 0.f ? d : 0.f;
  }
}

// bf16 halves of a packed pair, and the pair's sum of squares in one
// v_dot2_f32_bf16 (the products of bf16 values are exact in fp32).
__device__ __forceinline__ float bf_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf_hi(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }
__device__ __forceinline__ float bf_sq2(uint32_t w) {
  const bf16x2_t a = __builtin_bit_cast(bf16x2_t, w);
  return __builtin_amdgcn_fdot2_f32_bf16(a, a, 0.f, false);
}

// LRN of channels c0 .. c0+7 of pixel px (C channels, c0 % 8 == 0).  For bf16
// and the 5-channel window the window sums are built from pair sums of
// squares of the packed data: channel c's window c-2 .. c+2 is two pairs and
// one single.
template <typename T, int H, bool B075, int C>
__device__ __forceinline__ void lrn_unit(const T* px, int c0, float k, float alpha, float beta, float* o) {
  if constexpr (std::is_same<T, bf16>::value && H == 2) {
    uint32_t W[6];   // W[j] = channels (c0 - 2 + 2j, c0 - 1 + 2j)
    W[0] = c0 >= 8 ? *reinterpret_cast<const uint32_t*>(px + c0 - 2) : 0u;
    const uint4 q = *reinterpret_cast<const uint4*>(px + c0);
    W[1] = q.x; W[2] = q.y; W[3] = q.z; W[4] = q.w;
    W[5] = c0 + 8 < C ? *reinterpret_cast<const uint32_t*>(px + c0 + 8) : 0u;
    float Q[6];
#pragma unroll
    for (int j = 0; j < 6; ++j) Q[j] = bf_sq2(W[j]);
#pragma unroll
    for (int m = 0; m < 4; ++m) {
      const float ae = bf_lo(W[m + 2]), ao = bf_hi(W[m]);
      const float se = fmaf(ae, ae, Q[m] + Q[m + 1]);      // channels c0+2m-2 .. c0+2m+2
      const float so = fmaf(ao, ao, Q[m + 1] + Q[m + 2]);  // channels c0+2m-1 .. c0+2m+3
      float p, unused;
      lrn_pows<B075>(k + alpha * se, beta, p, unused);
      o[2 * m] = bf_lo(W[m + 1]) * p;
      lrn_pows<B075>(k + alpha * so, beta, p, unused);
      o[2 * m + 1] = bf_hi(W[m + 1]) * p;
    }
  } else {
    float v[24];
#pragma unroll
    for (int h = 0; h < 3; ++h) {
      const int cc = c0 + (h - 1) * 8;
      if (cc >= 0 && cc < C) Pack8<T>::load(px + cc, v + h * 8);
      else {
#pragma unroll
        for (int e = 0; e < 8; ++e) v[h * 8 + e] = 0.f;
      }
    }
    lrn8<H, B075>(v, k, alpha, beta, o);
  }
}

// LRN backward with the ReLU mask for channels c0 .. c0+7 of one pixel: apx
// holds the LRN input a and gpx the gradient g w.r.t. the LRN output.
template <typename T, int H, bool B075, int C>
__device__ __forceinline__ void lrn_bwd_unit(const T* apx, const T* gpx, int c0, float k, float alpha, float beta,
                                             float* o) {
  if constexpr (std::is_same<T, bf16>::value && H == 2) {
    uint32_t A[8];   // A[j] = a over channels (c0 - 4 + 2j, c0 - 3 + 2j)
    uint32_t G[6];   // G[j] = g over channels (c0 - 2 + 2j, c0 - 1 + 2j)
    if (c0 >= 8) {
      const uint2 l = *reinterpret_cast<const uint2*>(apx + c0 - 4);
      A[0] = l.x; A[1] = l.y;
      G[0] = *reinterpret_cast<const uint32_t*>(gpx + c0 - 2);
    } else {
      A[0] = A[1] = G[0] = 0u;
    }
    const uint4 aq = *reinterpret_cast<const uint4*>(apx + c0);
    const uint4 gq = *reinterpret_cast<const uint4*>(gpx + c0);
    A[2] = aq.x; A[3] = aq.y; A[4] = aq.z; A[5] = aq.w;
    G[1] = gq.x; G[2] = gq.y; G[3] = gq.z; G[4] = gq.w;
    if (c0 + 8 < C) {
      const uint2 h = *reinterpret_cast<const uint2*>(apx + c0 + 8);
      A[6] = h.x; A[7] = h.y;
      G[5] = *reinterpret_cast<const uint32_t*>(gpx + c0 + 8);
    } else {
      A[6] = A[7] = G[5] = 0u;
    }
    float Q[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) Q[j] = bf_sq2(A[j]);
    // positions r = 0..11: channels c0 - 2 + r (the reach of the 8 outputs' windows)
    float pb[12], tt[12];
#pragma unroll
    for (int r = 0; r < 12; ++r) {
      const int j = r >> 1;
      float s, ac, gc;
      if ((r & 1) == 0) {
        const float x = bf_lo(A[j + 2]);
        s = fmaf(x, x, Q[j] + Q[j + 1]);
        ac = bf_lo(A[j + 1]);
        gc = bf_lo(G[j]);
      } else {
        const float x = bf_hi(A[j]);
        s = fmaf(x, x, Q[j + 1] + Q[j + 2]);
        ac = bf_hi(A[j + 1]);
        gc = bf_hi(G[j]);
      }
      float p, qq;
      lrn_pows<B075>(k + alpha * s, beta, p, qq);
      pb[r] = p;
      tt[r] = gc * ac * qq;
    }
    const float c2 = 2.f * alpha * beta;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      float cross = 0.f;
#pragma unroll
      for (int j = 0; j < 5; ++j) cross += tt[i + j];
      const uint32_t aw = A[2 + (i >> 1)], gw = G[1 + (i >> 1)];
      const float aj = (i & 1) ? bf_hi(aw) : bf_lo(aw), gj = (i & 1) ? bf_hi(gw) : bf_lo(gw);
      const float d = gj * pb[i + 2] - c2 * aj * cross;
      o[i] = aj > 0.f ? d : 0.f;
    }
  } else {
    float av[24], gv[24];
#pragma unroll
    for (int hh = 0; hh < 3; ++hh) {
      const int cc = c0 + (hh - 1) * 8;
      if (cc >= 0 && cc < C) {
        Pack8<T>::load(apx + cc, av + hh * 8);
        Pack8<T>::load(gpx + cc, gv + hh * 8);
      } else {
#pragma unroll
        for (int e = 0; e < 8; ++e) { av[hh * 8 + e] = 0.f; gv[hh * 8 + e] = 0.f; }
      }
    }
    lrn_bwd8<H, B075>(av, gv, k, alpha, beta, o);
  }
}

// LRN followed by the overlapping 3x3 / stride-2 max-pool with argmax, fused:
// the LRN output is kept only in LDS (rounded to T exactly as a stored tensor
// would be), so pooled values and argmax equal those of the two separate
// steps.  One workgroup per (image n, pair of pooled rows i0 = 2 p, i0 + 1,
// channel group: see lrnpool_cg) over input rows 2 i0 .. 2 i0 + 4 (Hin =
// 2 Ho + 1; the last pair of an odd Ho has one pooled row and three input
// rows):
//   1. those rows (one contiguous run of NHWC; with channel groups, each
//      pixel's group and halo) are copied into LDS with direct-to-LDS loads
//      (one wait);
//   2. each thread normalises its (row, column, 8-channel) units from LDS into
//      registers, packed as stored, and, after a barrier, writes them back in
//      place;
//   3. the pooled rows and their argmax are taken from LDS.
// For bf16 the window maximum is taken on integer keys (value bits << 16 |
// 15 - d): the inputs are ReLU outputs, so every LRN output is >= +0 and its
// bf16 bits order as its value, and the key's low bits make the first of equal
// maxima in row-major scan order win, as in the float comparison.
// `dbg`, if not null, receives the LRN output of the rows the workgroup owns
// (2 i0 .. 2 i0 + 3, and the image's last row).  Workgroups are remapped so
// that the pairs of one image, which share an input row, run on one XCD.
constexpr int LRNPOOL_TPB = 512;

// Eight values of T packed as a stored tensor holds them (bf16: one 16-byte
// word, fp32: two), rounded as Pack8<T>::store rounds.
template <typename T> struct Packed8 { uint4 q[sizeof(T) / 2]; };
template <typename T>
__device__ __forceinline__ Packed8<T> pack8(const float* v) {
  Packed8<T> o;
  if constexpr (std::is_same<T, bf16>::value) {
    o.q[0] = make_uint4(f2bf2(v[0], v[1]), f2bf2(v[2], v[3]), f2bf2(v[4], v[5]), f2bf2(v[6], v[7]));
  } else {
    o.q[0] = make_uint4(__float_as_uint(v[0]), __float_as_uint(v[1]), __float_as_uint(v[2]), __float_as_uint(v[3]));
    o.q[1] = make_uint4(__float_as_uint(v[4]), __float_as_uint(v[5]), __float_as_uint(v[6]), __float_as_uint(v[7]));
  }
  return o;
}
template <typename T>
__device__ __forceinline__ void store8(T* p, const Packed8<T>& o) {
#pragma unroll
  for (int i = 0; i < (int)(sizeof(T) / 2); ++i) reinterpret_cast<uint4*>(p)[i] = o.q[i];
}

// Channels per workgroup of the fused LRN/pool (CG of the layer's C): a layer
// whose five-row tile of all channels leaves room for fewer than three
// workgroups per CU is split into channel groups of 128, each staged with an
// 8-channel halo on both sides (the LRN window reaches H <= 4 channels), so
// that four fit: layer 2 (27 x 256) 69 KB -> 39 KB.
template <typename T, int Win, int C>
constexpr int lrnpool_cg() {
  return 160 * 1024 / (5 * Win * C * (int)sizeof(T)) < 3 && C % 128 == 0 && C > 128 ? 128 : C;
}

// LRN of rows 0 .. nrows-1 of the LDS tile, in place: every thread computes
// its (row, column, 8-channel) units from LDS into packed registers (a unit
// past the end recomputes the last one, so no thread branches around the
// arithmetic), then, after a barrier, writes them back.  The tile holds the
// workgroup's channels cg0 .. cg0 + CG - 1 of each pixel at a pixel stride of
// PS values, channel c at offset c - cg0 + HALO (HALO = 8 with channel groups,
// else 0); lrn_unit's bounds use the layer's C.
template <typename T, int H, bool B075, int Win, int C>
__device__ __forceinline__ void lrn_pool_rows(T* rows, int nrows, int cg0, T* __restrict__ dbg, size_t dbg_row0,
                                              int own_last, float k, float alpha, float beta) {
  constexpr int CG = lrnpool_cg<T, Win, C>(), HALO = CG < C ? 8 : 0, PS = CG + 2 * HALO;
  constexpr int cpp = CG / 8, rowu = Win * cpp;
  constexpr int UPT = (5 * rowu + LRNPOOL_TPB - 1) / LRNPOOL_TPB;
  const int tid = threadIdx.x;
  const int units = nrows * rowu;
  Packed8<T> o[UPT];
#pragma unroll
  for (int t = 0; t < UPT; ++t) {
    const int u = min(tid + t * LRNPOOL_TPB, units - 1);
    const int pix = u / cpp, c0 = cg0 + (u - pix * cpp) * 8;
    float r[8];
    lrn_unit<T, H, B075, C>(rows + pix * PS + HALO - cg0, c0, k, alpha, beta, r);
    o[t] = pack8<T>(r);
  }
  __syncthreads();
#pragma unroll
  for (int t = 0; t < UPT; ++t) {
    const int u = tid + t * LRNPOOL_TPB;
    if (u < units) {
      const int pix = u / cpp, cl = (u - pix * cpp) * 8;
      store8<T>(rows + pix * PS + HALO + cl, o[t]);
      const int rr = pix / Win;
      if (dbg && (rr < 4 || own_last)) store8<T>(dbg + dbg_row0 + (size_t)pix * C + cg0 + cl, o[t]);
    }
  }
}

template <typename T, int H, bool B075, int Win, int C>
__global__ void __launch_bounds__(LRNPOOL_TPB) k_lrn_pool(const T* __restrict__ a, T* __restrict__ y,
                                                          uint8_t* __restrict__ arg, T* __restrict__ dbg,
                                                          float k, float alpha, float beta) {
  constexpr int Hin = Win, Ho = (Win - 1) / 2, Wo = Ho, NP = (Ho + 1) / 2;
  constexpr int CG = lrnpool_cg<T, Win, C>(), NG = C / CG, HALO = CG < C ? 8 : 0, PS = CG + 2 * HALO;
  static_assert(C % 8 == 0 && Hin == 2 * Ho + 1 && C % CG == 0, "fused LRN/pool geometry");
  constexpr int LDS_BYTES = ((5 * Win * PS * (int)sizeof(T) + 1023) / 1024) * 1024;
  __shared__ __attribute__((aligned(16))) char lds[LDS_BYTES];
  T* rows = reinterpret_cast<T*>(lds);
  const int nb = gridDim.x, xcd = blockIdx.x & 7, q = nb >> 3, rq = nb & 7;
  const int b = xcd * q + (xcd < rq ? xcd : rq) + (blockIdx.x >> 3);
  const int bp = b / NG, cg0 = (b - bp * NG) * CG;
  const int n = bp / NP, i0 = (bp - n * NP) * 2;
  const int npool = min(2, Ho - i0), nrows = 2 * npool + 1;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const size_t img = (size_t)Hin * Win * C;
  // 1. input rows 2 i0 .. 2 i0 + nrows - 1 -> LDS (1 KB per wave instruction; past the image reads as zero)
  {
    const __amdgpu_buffer_rsrc_t rs = buf_rsrc(a + n * img, (uint32_t)(img * sizeof(T)));
    const uint32_t base = (uint32_t)((size_t)2 * i0 * Win * C * sizeof(T));
    if constexpr (NG == 1) {
      // the rows are one contiguous run of NHWC
      const int nins = (nrows * Win * C * (int)sizeof(T) + 1023) / 1024;
      for (int j = wave; j < nins; j += LRNPOOL_TPB / 64)
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (lds_void_t*)(lds + j * 1024), 16,
                                                 (int)(base + j * 1024 + lane * 16), 0, 0, 0);
    } else {
      // each pixel's PS channels cg0 - 8 .. cg0 + CG + 7 as 16-byte granules,
      // laid out one after the other; a granule before the image's first
      // value (wrapped offset) or past its end reads as zero, and halo
      // channels of a neighbouring pixel are read but never used
      constexpr int GPP = PS * (int)sizeof(T) / 16;   // granules per pixel
      const int ng = nrows * Win * GPP, nins = (ng + 63) / 64;
      for (int j = wave; j < nins; j += LRNPOOL_TPB / 64) {
        const int g = min(j * 64 + lane, ng - 1);      // lanes past the end fetch the last granule again, into the tile's padding
        const int pix = g / GPP, gi = g - pix * GPP;
        const int64_t off = (int64_t)base + ((int64_t)pix * C + cg0 - HALO) * (int)sizeof(T) + gi * 16;
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (lds_void_t*)(lds + j * 1024), 16,
                                                 (int)(uint32_t)off, 0, 0, 0);
      }
    }
    wait_vmcnt<0>();
    __syncthreads();
  }
  // 2. LRN in place
  const size_t dbg_row0 = ((size_t)n * Hin + 2 * i0) * Win * C;
  const int own_last = 2 * i0 + nrows == Hin;
  lrn_pool_rows<T, H, B075, Win, C>(rows, nrows, cg0, dbg, dbg_row0, own_last, k, alpha, beta);
  __syncthreads();
  // 3. pool: pooled row i0 + ii from LDS rows 2 ii .. 2 ii + 2, columns 2j .. 2j+2
  constexpr int cpp = CG >> 3;
  for (int u = tid; u < npool * Wo * cpp; u += LRNPOOL_TPB) {
    const int ii = u / (Wo * cpp), ju = u - ii * (Wo * cpp);
    const int j = ju / cpp, cl = (ju - j * cpp) * 8, c0 = cg0 + cl;
    const T* px = rows + ((2 * ii) * Win + 2 * j) * PS + HALO + cl;
    const size_t og = (((size_t)n * Ho + i0 + ii) * Wo + j) * C + c0;
    uint32_t bi[8];
    if constexpr (std::is_same<T, bf16>::value) {
      uint32_t key[8];
#pragma unroll
      for (int d = 0; d < 9; ++d) {
        const int dy = d / 3, dx = d % 3;
        const uint4 qv = *reinterpret_cast<const uint4*>(px + (dy * Win + dx) * PS);
        const uint32_t w[4] = {qv.x, qv.y, qv.z, qv.w};
        const uint32_t code = 15u - (uint32_t)d;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const uint32_t klo = (w[e] << 16) | code, khi = (w[e] & 0xFFFF0000u) | code;
          key[2 * e] = d == 0 ? klo : max(key[2 * e], klo);
          key[2 * e + 1] = d == 0 ? khi : max(key[2 * e + 1], khi);
        }
      }
      uint32_t ow[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) ow[e] = (key[2 * e] >> 16) | (key[2 * e + 1] & 0xFFFF0000u);
#pragma unroll
      for (int e = 0; e < 8; ++e) bi[e] = 15u - (key[e] & 15u);
      *reinterpret_cast<uint4*>(y + og) = make_uint4(ow[0], ow[1], ow[2], ow[3]);
    } else {
      float best[8], v[8];
      Pack8<T>::load(px, best);
#pragma unroll
      for (int e = 0; e < 8; ++e) bi[e] = 0;
#pragma unroll
      for (int d = 1; d < 9; ++d) {
        const int dy = d / 3, dx = d % 3;
        Pack8<T>::load(px + (dy * Win + dx) * PS, v);
#pragma unroll
        for (int e = 0; e < 8; ++e)
          if (v[e] > best[e]) { best[e] = v[e]; bi[e] = d; }
      }
      Pack8<T>::store(y + og, best);
    }
    *reinterpret_cast<uint2*>(arg + og) = make_uint2(bi[0] | (bi[1] << 8) | (bi[2] << 16) | (bi[3] << 24),
                                                     bi[4] | (bi[5] << 8) | (bi[6] << 16) | (bi[7] << 24));
  }
}

// Max-pool backward (3x3 / stride 2, argmax codes dy*3+dx) for channels
// c0 .. c0+7 of the input pixels (h, 2m) and (h, 2m + 1): each one's sum,
// over the windows (i, j) that contain it and whose argmax it is, of
// dy[i][j] -- windows in row-major order -- rounded to T as a stored
// gradient would be.  Window column m - 1 reaches pixel 2m (dx = 2) only;
// window column m reaches pixel 2m (dx = 0) and 2m + 1 (dx = 1); window rows
// are ilo .. ihi (at most two, the same for the whole input row h).  Taking
// the pixels in pairs loads each window once and skips the windows that
// cannot contain a pixel.  dyL / argL hold pooled rows ilo .. ihi of the
// image, [row][j][c].
template <typename T, int C, int Wo>
__device__ __forceinline__ void pool_bwd_pair_lds(const T* dyL, const uint8_t* argL, int h, int m, int c0, int ilo,
                                                  int ihi, Packed8<T>& g0, Packed8<T>& g1) {
  float acc0[8], acc1[8];
#pragma unroll
  for (int q = 0; q < 8; ++q) acc0[q] = acc1[q] = 0.f;
#pragma unroll
  for (int di = 0; di < 2; ++di) {
    const int i = ilo + di;
    if (i > ihi) break;   // uniform over the workgroup
    const uint32_t row_code = (uint32_t)(h - 2 * i) * 3u;
    float g[8];
    if (m >= 1) {   // window (i, m - 1)
      const int off = (di * Wo + m - 1) * C + c0;
      const uint2 am = *reinterpret_cast<const uint2*>(argL + off);
      Pack8<T>::load(dyL + off, g);
#pragma unroll
      for (int q = 0; q < 8; ++q) {
        const uint32_t bq = ((q < 4 ? am.x : am.y) >> ((q & 3) * 8)) & 0xFFu;
        if (bq == row_code + 2u) acc0[q] += g[q];
      }
    }
    if (m < Wo) {   // window (i, m)
      const int off = (di * Wo + m) * C + c0;
      const uint2 am = *reinterpret_cast<const uint2*>(argL + off);
      Pack8<T>::load(dyL + off, g);
#pragma unroll
      for (int q = 0; q < 8; ++q) {
        const uint32_t bq = ((q < 4 ? am.x : am.y) >> ((q & 3) * 8)) & 0xFFu;
        if (bq == row_code) acc0[q] += g[q];
        if (bq == row_code + 1u) acc1[q] += g[q];
      }
    }
  }
  g0 = pack8<T>(acc0);
  g1 = pack8<T>(acc1);
}

// Max-pool backward, LRN backward and the ReLU mask in one pass.  One
// workgroup per input row (image n, row h) of a Win x C layer:
//   1. the row of the LRN input a, and the one or two pooled rows of dy and
//      argmax whose windows cover row h, are copied into LDS with
//      direct-to-LDS loads, all issued before one wait;
//   2. each thread forms the pooled gradient g (w.r.t. the LRN output) of its
//      (pair of columns, 8-channel) units from LDS, rounded as a stored
//      gradient would be, into a third LDS row;
//   3. each unit's LRN backward reads its channel neighbours of a and g from
//      LDS, applies the ReLU mask and writes da.
// da therefore equals that of the separate steps.  `dbg`, if not null,
// receives g.  `brow`, if not null, receives the row's column sums of da as
// stored (the bias gradient's share of the row): the stored units go back
// into LDS, eight threads' runs of pixels per channel group are summed, then
// the eight runs in order.
constexpr int PLB_TPB = 512;   // eight waves per row: more loads in flight per LDS byte than four
template <typename T, int H, bool B075, int Win, int C>
__global__ void __launch_bounds__(PLB_TPB) k_pool_lrn_bwd(const T* __restrict__ dy, const uint8_t* __restrict__ arg,
                                                      const T* __restrict__ a, T* __restrict__ da,
                                                      T* __restrict__ dbg, float* __restrict__ brow, float k,
                                                      float alpha, float beta) {
  constexpr int Hin = Win, Ho = (Win - 1) / 2, Wo = Ho, cpp = C / 8, units = Win * cpp;
  constexpr int UPT = (units + PLB_TPB - 1) / PLB_TPB;   // units per thread
  static_assert(C % 8 == 0, "pool/LRN backward geometry");
  constexpr int KB = 1024;
  constexpr int ROW_BYTES = (Win * C * (int)sizeof(T) + KB - 1) / KB * KB;
  constexpr int DY_BYTES = (2 * Wo * C * (int)sizeof(T) + KB - 1) / KB * KB;
  constexpr int ARG_BYTES = (2 * Wo * C + KB - 1) / KB * KB;
  __shared__ __attribute__((aligned(16))) char lds[2 * ROW_BYTES + DY_BYTES + ARG_BYTES];
  T* arow = reinterpret_cast<T*>(lds);
  T* grow = reinterpret_cast<T*>(lds + ROW_BYTES);
  const T* dyL = reinterpret_cast<const T*>(lds + 2 * ROW_BYTES);
  const uint8_t* argL = reinterpret_cast<const uint8_t*>(lds + 2 * ROW_BYTES + DY_BYTES);
  const int nb = gridDim.x, xcd = blockIdx.x & 7, q = nb >> 3, rq = nb & 7;
  const int b = xcd * q + (xcd < rq ? xcd : rq) + (blockIdx.x >> 3);
  const int n = b / Hin, h = b - n * Hin;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const size_t row0 = ((size_t)n * Hin + h) * Win * C;   // element offset of the row
  // pooled rows whose windows (rows 2i .. 2i+2) contain row h
  const int ilo = h >= 2 ? (h - 1) / 2 : 0, ihi = min(h / 2, Ho - 1);
  {
    // descriptors bound each copy to its rows; the rest of an LDS region reads zero
    const size_t prow = ((size_t)n * Ho + ilo) * Wo * C;
    const uint32_t pel = (uint32_t)((ihi - ilo + 1) * Wo * C);
    const __amdgpu_buffer_rsrc_t ra = buf_rsrc(a + row0, (uint32_t)(Win * C * sizeof(T)));
    const __amdgpu_buffer_rsrc_t rd = buf_rsrc(dy + prow, pel * (uint32_t)sizeof(T));
    const __amdgpu_buffer_rsrc_t rg = buf_rsrc(arg + prow, pel);
    for (int j = wave; j < ROW_BYTES / KB; j += PLB_TPB / 64)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(ra, (lds_void_t*)(lds + j * KB), 16, j * KB + lane * 16, 0, 0, 0);
    for (int j = wave; j < DY_BYTES / KB; j += PLB_TPB / 64)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rd, (lds_void_t*)(lds + 2 * ROW_BYTES + j * KB), 16,
                                               j * KB + lane * 16, 0, 0, 0);
    for (int j = wave; j < ARG_BYTES / KB; j += PLB_TPB / 64)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rg, (lds_void_t*)(lds + 2 * ROW_BYTES + DY_BYTES + j * KB), 16,
                                               j * KB + lane * 16, 0, 0, 0);
    wait_vmcnt<0>();
    __syncthreads();
  }
  // 2. pooled gradient, a pair of columns per (unit, 8 channels)
  constexpr int pair_units = (Win + 1) / 2 * cpp;
#pragma unroll
  for (int t = 0; t < (pair_units + PLB_TPB - 1) / PLB_TPB; ++t) {
    const int u = tid + t * PLB_TPB;
    if (u < pair_units) {
      const int m = u / cpp, c0 = (u - m * cpp) * 8;
      Packed8<T> g0, g1;
      pool_bwd_pair_lds<T, C, Wo>(dyL, argL, h, m, c0, ilo, ihi, g0, g1);
      store8<T>(grow + 2 * m * C + c0, g0);
      if (dbg) store8<T>(dbg + row0 + 2 * m * C + c0, g0);
      if (2 * m + 1 < Win) {
        store8<T>(grow + (2 * m + 1) * C + c0, g1);
        if (dbg) store8<T>(dbg + row0 + (2 * m + 1) * C + c0, g1);
      }
    }
  }
  __syncthreads();
  Packed8<T> od[UPT];
#pragma unroll
  for (int t = 0; t < UPT; ++t) {
    const int u = tid + t * PLB_TPB;
    if (u < units) {
      const int w = u / cpp, c0 = (u - w * cpp) * 8;
      float o[8];
      lrn_bwd_unit<T, H, B075, C>(arow + w * C, grow + w * C, c0, k, alpha, beta, o);
      od[t] = pack8<T>(o);
      store8<T>(da + row0 + w * C + c0, od[t]);
    }
  }
  if (brow) {   // uniform
    constexpr int S = 8, L = (Win + S - 1) / S;   // runs of pixels per channel group
    static_assert(S * C * 4 <= DY_BYTES + ARG_BYTES, "run sums fit the pooled-row staging");
    float* runs = reinterpret_cast<float*>(lds + 2 * ROW_BYTES);   // [S][C], over the staging no longer read
    __syncthreads();   // every unit's channel neighbours have been read from arow and grow
#pragma unroll
    for (int t = 0; t < UPT; ++t) {
      const int u = tid + t * PLB_TPB;
      if (u < units) store8<T>(arow + u * 8, od[t]);   // unit u = (w, c0) sits at w * C + c0
    }
    __syncthreads();
    if (tid < S * cpp) {
      const int s = tid / cpp, c0 = (tid - s * cpp) * 8;
      float acc[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) acc[e] = 0.f;
      for (int w = s * L; w < min(Win, s * L + L); ++w) {
        float v[8];
        Pack8<T>::load(arow + w * C + c0, v);
#pragma unroll
        for (int e = 0; e < 8; ++e) acc[e] += v[e];
      }
#pragma unroll
      for (int e = 0; e < 8; ++e) runs[s * C + c0 + e] = acc[e];
    }
    __syncthreads();
    for (int c = tid; c < C; c += PLB_TPB) {
      float sum = 0.f;
#pragma unroll
      for (int s = 0; s < S; ++s) sum += runs[s * C + c];
      brow[((size_t)n * Hin + h) * C + c] = sum;
    }
  }
}

// Calls fn.operator()<H, B075>() for the window half-width and beta.
template <class Fn>
static hipError_t lrn_dispatch(int half, float beta, Fn&& fn) {
  const bool b075 = beta == 0.75f;
#define AX_LRN_CASE(HH) \
  case HH: return b075 ? fn.template operator()<HH, true>() : fn.template operator()<HH, false>();
  switch (half) {
    AX_LRN_CASE(0) AX_LRN_CASE(1) AX_LRN_CASE(2) AX_LRN_CASE(3) AX_LRN_CASE(4)
    default: return hipErrorInvalidValue;
  }
#undef AX_LRN_CASE
}

template <typename T, int Win, int C>
struct LrnPoolFn {
  const void* a; void* y; uint8_t* arg; void* dbg; int N; float k, alpha, beta; hipStream_t st;
  template <int H, bool B075>
  hipError_t operator()() const {
    constexpr int Ho = (Win - 1) / 2, NG = C / lrnpool_cg<T, Win, C>();
    hipLaunchKernelGGL((k_lrn_pool<T, H, B075, Win, C>), dim3(N * ((Ho + 1) / 2) * NG), dim3(LRNPOOL_TPB), 0, st,
                       (const T*)a,
                       (T*)y, arg, (T*)dbg, k, alpha, beta);
    return hipGetLastError();
  }
};
template <typename T, int Win, int C>
struct PoolLrnBwdFn {
  const void* dy; const uint8_t* arg; const void* a; void* da; void* dbg; float* brow; int N; float k, alpha, beta;
  hipStream_t st;
  template <int H, bool B075>
  hipError_t operator()() const {
    hipLaunchKernelGGL((k_pool_lrn_bwd<T, H, B075, Win, C>), dim3(N * Win), dim3(PLB_TPB), 0, st, (const T*)dy, arg,
                       (const T*)a, (T*)da, (T*)dbg, brow, k, alpha, beta);
    return hipGetLastError();
  }
};

hipError_t lrn_pool_fwd(DType dt, const void* a, void* y, uint8_t* arg, void* dbg, int N, int H, int W, int C,
                        float k, float alpha, float beta, int n, hipStream_t st, const KTimer* kt) {
  // the two layers of the network: 55 x 55 x 96 and 27 x 27 x 256
  const int layer = (H == 55 && W == 55 && C == 96) ? 1 : (H == 27 && W == 27 && C == 256) ? 2 : 0;
  if (!layer) return hipErrorInvalidValue;
  rec_start(kt, st);
  hipError_t e;
  if (layer == 1)
    e = dt == BF16 ? lrn_dispatch(n / 2, beta, LrnPoolFn<bf16, 55, 96>{a, y, arg, dbg, N, k, alpha, beta, st})
                   : lrn_dispatch(n / 2, beta, LrnPoolFn<float, 55, 96>{a, y, arg, dbg, N, k, alpha, beta, st});
  else
    e = dt == BF16 ? lrn_dispatch(n / 2, beta, LrnPoolFn<bf16, 27, 256>{a, y, arg, dbg, N, k, alpha, beta, st})
                   : lrn_dispatch(n / 2, beta, LrnPoolFn<float, 27, 256>{a, y, arg, dbg, N, k, alpha, beta, st});
  rec_stop(kt, st);
  return e;
}


hipError_t pool_lrn_bwd(DType dt, const void* dy, const uint8_t* arg, const void* a, void* da, void* dbg,
                        float* bias_rows, int N, int H, int W, int C, float k, float alpha, float beta, int n,
                        hipStream_t st, const KTimer* kt) {
  // the two layers of the network: 55 x 55 x 96 and 27 x 27 x 256
  const int layer = (H == 55 && W == 55 && C == 96) ? 1 : (H == 27 && W == 27 && C == 256) ? 2 : 0;
  if (!layer) return hipErrorInvalidValue;
  rec_start(kt, st);
  hipError_t e;
  if (layer == 1)
    e = dt == BF16
            ? lrn_dispatch(n / 2, beta, PoolLrnBwdFn<bf16, 55, 96>{dy, arg, a, da, dbg, bias_rows, N, k, alpha, beta, st})
            : lrn_dispatch(n / 2, beta,
                           PoolLrnBwdFn<float, 55, 96>{dy, arg, a, da, dbg, bias_rows, N, k, alpha, beta, st});
  else
    e = dt == BF16
            ? lrn_dispatch(n / 2, beta,
                           PoolLrnBwdFn<bf16, 27, 256>{dy, arg, a, da, dbg, bias_rows, N, k, alpha, beta, st})
            : lrn_dispatch(n / 2, beta,
                           PoolLrnBwdFn<float, 27, 256>{dy, arg, a, da, dbg, bias_rows, N, k, alpha, beta, st});
  rec_stop(kt, st);
  return e;
}

// =========================================================================
// Overlapping max-pool 3x3 / stride 2, NHWC, with argmax (dy*3 + dx of the
// first maximum in a row-major scan of the window)
// =========================================================================
// Pool 5: max-pool whose output is flattened in (c, h, w) order for FC6.
// One workgroup per (image n, 32-channel block): one thread per (position,
// 8-channel) unit takes its window's maximum and argmax; the pooled values go
// to LDS as [c][h*Wo+w], which is exactly the block's contiguous run of the
// flat output.  For bf16 the maximum is taken on integer keys (value bits <<
// 16 | 15 - d), valid because the input is a ReLU output (every value >= +0,
// so bf16 bits order as values); equal maxima resolve to the first in
// row-major scan order, as in the float comparison.
constexpr int POOL5_CB = 32;    // channels per workgroup
constexpr int POOL5_P = 64;     // max pooled positions (Ho * Wo)

// max/argmax of the 3x3 window at px (row stride W*C elements) for 8 channels
template <typename T>
__device__ __forceinline__ void pool_window8(const T* px, int64_t rs, int C, float* best, uint32_t* bi) {
  if constexpr (std::is_same<T, bf16>::value) {
    uint32_t key[8];
#pragma unroll
    for (int d = 0; d < 9; ++d) {
      const uint4 q = *reinterpret_cast<const uint4*>(px + (d / 3) * rs + (d % 3) * C);
      const uint32_t w[4] = {q.x, q.y, q.z, q.w};
      const uint32_t code = 15u - (uint32_t)d;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const uint32_t klo = (w[e] << 16) | code, khi = (w[e] & 0xFFFF0000u) | code;
        key[2 * e] = d == 0 ? klo : max(key[2 * e], klo);
        key[2 * e + 1] = d == 0 ? khi : max(key[2 * e + 1], khi);
      }
    }
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      best[e] = __uint_as_float(key[e] & 0xFFFF0000u);
      bi[e] = 15u - (key[e] & 15u);
    }
  } else {
    float v[8];
    Pack8<T>::load(px, best);
#pragma unroll
    for (int e = 0; e < 8; ++e) bi[e] = 0;
#pragma unroll
    for (int d = 1; d < 9; ++d) {
      Pack8<T>::load(px + (d / 3) * rs + (d % 3) * C, v);
#pragma unroll
      for (int e = 0; e < 8; ++e)
        if (v[e] > best[e]) { best[e] = v[e]; bi[e] = d; }
    }
  }
}

template <typename T>
__global__ void __launch_bounds__(TPB) k_pool5_fwd(const T* __restrict__ x, T* __restrict__ y,
                                                   uint8_t* __restrict__ arg, int H, int W, int C, int Ho,
                                                   int Wo) {
  __shared__ __attribute__((aligned(16))) T ly[POOL5_CB * POOL5_P];
  const int nblk = C / POOL5_CB, n = blockIdx.x / nblk, cb = blockIdx.x - n * nblk;
  const int P = Ho * Wo, units = P * (POOL5_CB / 8);
  const int u = threadIdx.x;
  if (u < units) {
    const int pos = u / (POOL5_CB / 8), ch8 = u - pos * (POOL5_CB / 8);
    const int i = pos / Wo, j = pos - i * Wo, c0 = cb * POOL5_CB + ch8 * 8;
    float best[8];
    uint32_t bi[8];
    pool_window8<T>(x + (((size_t)n * H + 2 * i) * W + 2 * j) * C + c0, (int64_t)W * C, C, best, bi);
    *reinterpret_cast<uint2*>(arg + (((size_t)n * Ho + i) * Wo + j) * C + c0) =
        make_uint2(bi[0] | (bi[1] << 8) | (bi[2] << 16) | (bi[3] << 24),
                   bi[4] | (bi[5] << 8) | (bi[6] << 16) | (bi[7] << 24));
#pragma unroll
    for (int e = 0; e < 8; ++e) ly[(ch8 * 8 + e) * P + pos] = Num<T>::store(best[e]);
  }
  __syncthreads();
  // the block's run of the flat output: POOL5_CB * P elements, 16-byte chunks
  T* out = y + (size_t)n * C * P + (size_t)cb * POOL5_CB * P;
  constexpr int V = 16 / sizeof(T);
  for (int q = threadIdx.x; q < POOL5_CB * P / V; q += TPB)
    *reinterpret_cast<uint4*>(out + q * V) = *reinterpret_cast<const uint4*>(ly + q * V);
}

// Pool-5 backward from the flat (c, h, w) gradient, times the ReLU mask of
// the pool input [mask > 0]: one workgroup per (image n, 32-channel block).
// The block's run of the flat gradient (POOL5_CB * P values) is read once in
// 4-element pieces and transposed into LDS as [h*Wo+w][c]; each thread then
// sums, for its (row, column, 8-channel) units, the windows whose argmax is
// the pixel (windows in row-major order).  Every global read of a thread (its
// gradient pieces, its units' argmax codes and mask rows) is issued before the
// first is used, so the thread waits one memory latency, not one per unit.
constexpr int POOL5_UIT = 4;   // units per thread: H W (POOL5_CB / 8) <= POOL5_UIT TPB (host-checked)
constexpr int POOL5_GIT = (POOL5_CB * POOL5_P / 4 + TPB - 1) / TPB;   // gradient pieces per thread

template <typename T>
__global__ void __launch_bounds__(TPB) k_pool5_bwd(const T* __restrict__ dy, const uint8_t* __restrict__ arg,
                                                   const T* __restrict__ mask, T* __restrict__ dx, int H, int W,
                                                   int C, int Ho, int Wo) {
  constexpr int LS = POOL5_CB + 8;   // padded row: the transposing writes spread over banks
  constexpr int CPP = POOL5_CB / 8;
  __shared__ __attribute__((aligned(16))) T lg[POOL5_P * LS];
  const int nblk = C / POOL5_CB, n = blockIdx.x / nblk, cb = blockIdx.x - n * nblk;
  const int P = Ho * Wo, pieces = POOL5_CB * P / 4, units = H * W * CPP;
  const T* src = dy + (size_t)n * C * P + (size_t)cb * POOL5_CB * P;
  // reads: indices past the end are clamped to the last valid one (a valid
  // address; those values are never used)
  T g4[POOL5_GIT][4];
#pragma unroll
  for (int it = 0; it < POOL5_GIT; ++it) {
    const int e4 = min((int)threadIdx.x + it * TPB, pieces - 1);
    if constexpr (sizeof(T) == 2) {
      const uint2 q = *reinterpret_cast<const uint2*>(src + e4 * 4);
      g4[it][0] = (T)(q.x & 0xFFFFu); g4[it][1] = (T)(q.x >> 16);
      g4[it][2] = (T)(q.y & 0xFFFFu); g4[it][3] = (T)(q.y >> 16);
    } else {
      const float4 q = *reinterpret_cast<const float4*>(src + e4 * 4);
      g4[it][0] = q.x; g4[it][1] = q.y; g4[it][2] = q.z; g4[it][3] = q.w;
    }
  }
  uint2 am[POOL5_UIT][4];
  float mk[POOL5_UIT][8];
#pragma unroll
  for (int it = 0; it < POOL5_UIT; ++it) {
    const int u = min((int)threadIdx.x + it * TPB, units - 1);
    const int hw = u / CPP, ch8 = u - hw * CPP, h = hw / W, w = hw - h * W;
    const int c0 = cb * POOL5_CB + ch8 * 8;
    const int i0 = h >= 2 ? (h - 1) / 2 : 0, j0 = w >= 2 ? (w - 1) / 2 : 0;
#pragma unroll
    for (int d = 0; d < 4; ++d) {
      const int i = min(i0 + (d >> 1), Ho - 1), j = min(j0 + (d & 1), Wo - 1);
      am[it][d] = *reinterpret_cast<const uint2*>(arg + (((size_t)n * Ho + i) * Wo + j) * C + c0);
    }
    Pack8<T>::load(mask + (((size_t)n * H + h) * W + w) * C + c0, mk[it]);
  }
#pragma unroll
  for (int it = 0; it < POOL5_GIT; ++it) {
    const int e4 = threadIdx.x + it * TPB;
    if (e4 < pieces) {
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        const int e = e4 * 4 + k, c = e / P, pos = e - c * P;
        lg[pos * LS + c] = g4[it][k];
      }
    }
  }
  __syncthreads();
#pragma unroll
  for (int it = 0; it < POOL5_UIT; ++it) {
    const int u = threadIdx.x + it * TPB;
    if (u >= units) break;
    const int hw = u / CPP, ch8 = u - hw * CPP, h = hw / W, w = hw - h * W;
    const int c0 = cb * POOL5_CB + ch8 * 8;
    const int i0 = h >= 2 ? (h - 1) / 2 : 0, i1 = min(h / 2, Ho - 1);
    const int j0 = w >= 2 ? (w - 1) / 2 : 0, j1 = min(w / 2, Wo - 1);
    float acc[8];
#pragma unroll
    for (int q = 0; q < 8; ++q) acc[q] = 0.f;
#pragma unroll
    for (int d = 0; d < 4; ++d) {
      const int i = i0 + (d >> 1), j = j0 + (d & 1);
      if (i <= i1 && j <= j1) {
        const uint32_t code = (uint32_t)((h - 2 * i) * 3 + (w - 2 * j));
        float g[8];
        Pack8<T>::load(lg + (i * Wo + j) * LS + ch8 * 8, g);
#pragma unroll
        for (int q = 0; q < 8; ++q) {
          const uint32_t b = ((q < 4 ? am[it][d].x : am[it][d].y) >> ((q & 3) * 8)) & 0xFFu;
          if (b == code) acc[q] += g[q];
        }
      }
    }
#pragma unroll
    for (int q = 0; q < 8; ++q) acc[q] = mk[it][q] > 0.f ? acc[q] : 0.f;
    Pack8<T>::store(dx + (((size_t)n * H + h) * W + w) * C + c0, acc);
  }
}

static bool pool5_shape_ok(int H, int W, int C, int& Ho, int& Wo) {
  Ho = (H - 3) / 2 + 1; Wo = (W - 3) / 2 + 1;
  return C % POOL5_CB == 0 && Ho * Wo <= POOL5_P && Ho * Wo * (POOL5_CB / 8) <= TPB &&
         (POOL5_CB * Ho * Wo) % 8 == 0 && H * W * (POOL5_CB / 8) <= POOL5_UIT * TPB;
}

hipError_t pool5_fwd(DType dt, const void* x, void* y, uint8_t* arg, int N, int H, int W, int C, hipStream_t st,
                     const KTimer* kt) {
  int Ho, Wo;
  if (!pool5_shape_ok(H, W, C, Ho, Wo)) return hipErrorInvalidValue;
  const dim3 g(N * (C / POOL5_CB));
  rec_start(kt, st);
  if (dt == BF16) hipLaunchKernelGGL((k_pool5_fwd<bf16>), g, dim3(TPB), 0, st, (const bf16*)x, (bf16*)y, arg, H, W, C, Ho, Wo);
  else hipLaunchKernelGGL((k_pool5_fwd<float>), g, dim3(TPB), 0, st, (const float*)x, (float*)y, arg, H, W, C, Ho, Wo);
  rec_stop(kt, st);
  return hipGetLastError();
}

hipError_t pool5_bwd(DType dt, const void* dy, const uint8_t* arg, const void* mask, void* dx, int N, int H,
                     int W, int C, hipStream_t st, const KTimer* kt) {
  int Ho, Wo;
  if (!pool5_shape_ok(H, W, C, Ho, Wo) || !mask) return hipErrorInvalidValue;
  const dim3 g(N * (C / POOL5_CB));
  rec_start(kt, st);
  if (dt == BF16) hipLaunchKernelGGL((k_pool5_bwd<bf16>), g, dim3(TPB), 0, st, (const bf16*)dy, arg, (const bf16*)mask, (bf16*)dx, H, W, C, Ho, Wo);
  else hipLaunchKernelGGL((k_pool5_bwd<float>), g, dim3(TPB), 0, st, (const float*)dy, arg, (const float*)mask, (float*)dx, H, W, C, Ho, Wo);
  rec_stop(kt, st);
  return hipGetLastError();
}

// =========================================================================
// Softmax, cross-entropy, ten-view mean: one wavefront per row
// =========================================================================
__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, 64));
  return v;
}
__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, 64);
  return v;
}

// Network head, one workgroup per row m: the FC8 split-K partials summed in
// split order plus the bias (the logits, stored fp32), then the softmax and,
// with CE, the cross-entropy gradient (p - onehot(y)) / M and the row's loss
// -(z_y - max - log sum exp).  Each thread holds 4 consecutive logits.
constexpr int HEAD_MAX_O = 4 * TPB;
template <typename T, bool CE>
__global__ void __launch_bounds__(TPB) k_fc_head(const float* __restrict__ part, int S, int M, int O,
                                                 const T* __restrict__ bias, float* __restrict__ logits,
                                                 const int32_t* __restrict__ labels, float* __restrict__ p,
                                                 T* __restrict__ dz, float* __restrict__ rowloss) {
  __shared__ float red[TPB / 64];
  const int m = blockIdx.x, t = threadIdx.x, lane = t & 63, wave = t >> 6;
  const int n0 = 4 * t;
  const bool on = n0 < O;
  float v[4] = {-INFINITY, -INFINITY, -INFINITY, -INFINITY};
  if (on) {
    float a[4] = {0.f, 0.f, 0.f, 0.f};
    for (int s2 = 0; s2 < S; ++s2) {
      const float4 q = *reinterpret_cast<const float4*>(part + ((int64_t)s2 * M + m) * O + n0);
      a[0] += q.x; a[1] += q.y; a[2] += q.z; a[3] += q.w;
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) v[i] = a[i] + Num<T>::load(bias[n0 + i]);
    *reinterpret_cast<float4*>(logits + (int64_t)m * O + n0) = make_float4(v[0], v[1], v[2], v[3]);
  }
  // row maximum, then the sum of exponentials: each wave reduces with
  // shuffles, then the waves' values combine in wave order
  float mx = fmaxf(fmaxf(v[0], v[1]), fmaxf(v[2], v[3]));
  mx = wave_max(mx);
  if (lane == 0) red[wave] = mx;
  __syncthreads();
  mx = red[0];
#pragma unroll
  for (int w = 1; w < TPB / 64; ++w) mx = fmaxf(mx, red[w]);
  __syncthreads();
  float e[4], s = 0.f;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    e[i] = on ? expf(v[i] - mx) : 0.f;
    s += e[i];
  }
  s = wave_sum(s);
  if (lane == 0) red[wave] = s;
  __syncthreads();
  s = red[0];
#pragma unroll
  for (int w = 1; w < TPB / 64; ++w) s += red[w];
  if (!on) return;
  const float inv = 1.f / s;
  int y = 0;
  if (CE) { y = labels[m]; y = y < 0 ? 0 : (y >= O ? O - 1 : y); }
  float pr[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) pr[i] = e[i] * inv;
  if (p) *reinterpret_cast<float4*>(p + (int64_t)m * O + n0) = make_float4(pr[0], pr[1], pr[2], pr[3]);
  if (CE) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      dz[(int64_t)m * O + n0 + i] = Num<T>::store((pr[i] - (n0 + i == y ? 1.f : 0.f)) / (float)M);
      if (n0 + i == y) rowloss[m] = -(v[i] - mx - logf(s));
    }
  }
}

template <typename T>
static hipError_t fc_head_t(int M, int K, int O, const void* x, const void* w, const void* b, float* logits,
                            const int32_t* labels, float* probs, void* dz, float* rowloss, float* part,
                            size_t part_bytes, hipStream_t st, const KTimer* kt) {
  if (O % 4 || O > HEAD_MAX_O) return hipErrorInvalidValue;
  int S = 1;
  hipError_t err = fc_partials<T>(M, K, O, x, w, part, part_bytes, st, kt, S);
  if (err != hipSuccess) return err;
  if (labels)
    hipLaunchKernelGGL((k_fc_head<T, true>), dim3(M), dim3(TPB), 0, st, part, S, M, O, (const T*)b, logits, labels,
                       probs, (T*)dz, rowloss);
  else
    hipLaunchKernelGGL((k_fc_head<T, false>), dim3(M), dim3(TPB), 0, st, part, S, M, O, (const T*)b, logits,
                       labels, probs, (T*)nullptr, (float*)nullptr);
  return hipGetLastError();
}

hipError_t fc_head(DType dt, int M, int K, int O, const void* x, const void* w, const void* b, float* logits,
                   const int32_t* labels, float* probs, void* dz, float* rowloss, float* part, size_t part_bytes,
                   hipStream_t st, const KTimer* kt) {
  return dt == BF16 ? fc_head_t<bf16>(M, K, O, x, w, b, logits, labels, probs, dz, rowloss, part, part_bytes, st, kt)
                    : fc_head_t<float>(M, K, O, x, w, b, logits, labels, probs, dz, rowloss, part, part_bytes, st, kt);
}

__global__ void k_view_mean(const float* __restrict__ p, float* __restrict__ out, int N, int O) {
  const int64_t t = (int64_t)blockIdx.x * TPB + threadIdx.x;
  if (t >= (int64_t)N * O) return;
  const int n = (int)(t / O), i = (int)(t - (int64_t)n * O);
  float s = 0.f;
#pragma unroll
  for (int v = 0; v < 10; ++v) s += p[((int64_t)n * 10 + v) * O + i];
  out[t] = s / 10.f;
}
hipError_t view_mean(const float* p, float* out, int N, int O, hipStream_t st) {
  hipLaunchKernelGGL(k_view_mean, grid1d((int64_t)N * O), dim3(TPB), 0, st, p, out, N, O);
  return hipGetLastError();
}

// =========================================================================
// Column sums
// =========================================================================
// Column sums of a row-major [rows][C] tensor (bias gradients: sum of dY over
// all pixels of the batch), in fp32, deterministic: block (b, j) sums rows
// [b*rb, (b+1)*rb) of columns [j*512, (j+1)*512) -- each thread a run of 8
// columns over every L-th row, L = 256 / (columns / 8), four rows in flight --
// and combines its L partial sums in a fixed order.  With one row block the
// result goes straight to `out`; otherwise a second pass adds the row blocks
// in order.
static constexpr int COLSUM_CW = 512;
// Row blocks per layer: all layers' blocks run in one launch, so 256 per
// layer fill the chip, and each bias element then sums at most 256 partials.
static int colsum_blocks(int64_t rows, int C) {
  const int ct = cdiv(C, COLSUM_CW);
  int64_t nb = (256 + ct - 1) / ct;
  nb = std::min<int64_t>(nb, (rows + 15) / 16);      // at least 16 rows per block
  return (int)std::max<int64_t>(nb, 1);
}

// Column sums of one (row block, column tile) of x[rows][C]: part[rowblock][c].
template <typename T>
__device__ __forceinline__ void colsum_block(const T* __restrict__ x, int64_t rows, int C, int64_t rb,
                                             int rowblock, int ctile, float* __restrict__ part) {
  __shared__ float sh[TPB][9];
  const int c0 = ctile * COLSUM_CW;
  const int w = min(COLSUM_CW, C - c0);
  const int cpr = w >> 3, nrl = TPB / cpr;
  const int t = threadIdx.x, cc = t % cpr, rl = t / cpr;
  const int64_t r0 = (int64_t)rowblock * rb, r1 = min(r0 + rb, rows);
  float acc[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) acc[e] = 0.f;
  if (rl < nrl) {
    const T* base = x + c0 + cc * 8;
    int64_t r = r0 + rl;
    for (; r + 3 * nrl < r1; r += 4 * nrl) {
      float v[4][8];
#pragma unroll
      for (int u = 0; u < 4; ++u) Pack8<T>::load(base + (r + u * nrl) * C, v[u]);
#pragma unroll
      for (int u = 0; u < 4; ++u)
#pragma unroll
        for (int e = 0; e < 8; ++e) acc[e] += v[u][e];
    }
    for (; r < r1; r += nrl) {
      float v[8];
      Pack8<T>::load(base + r * C, v);
#pragma unroll
      for (int e = 0; e < 8; ++e) acc[e] += v[e];
    }
  }
#pragma unroll
  for (int e = 0; e < 8; ++e) sh[t][e] = acc[e];
  __syncthreads();
  for (int col = t; col < w; col += TPB) {
    const int q = col >> 3, e = col & 7;
    float s = 0.f;
    for (int j = 0; j < nrl; ++j) s += sh[j * cpr + q][e];
    part[(int64_t)rowblock * C + c0 + col] = s;
  }
}

// Bias gradients of several layers, each the column sum of the layer's output
// gradient dy[rows][C] over its N*H*W rows, followed by the SGD update of the
// bias, in two launches:
//   1. every (layer, row block, column tile) block writes one partial row;
//   2. one workgroup per 32 consecutive bias elements of a layer sums their
//      partials (eight row groups, each over every eighth partial row in
//      order, then the eight group sums in order), stores the gradients and
//      updates the biases (fp32 master, momentum, and working copy).  A row
//      group reads 128 contiguous bytes of each partial row.
struct BiasArgs1 {
  const void* x[BIAS_MAX];
  float* part[BIAS_MAX];
  int64_t rows[BIAS_MAX], rb[BIAS_MAX];
  int C[BIAS_MAX], nb[BIAS_MAX], f32[BIAS_MAX];
  int bstart[BIAS_MAX + 1];
  int n;
};
struct BiasArgs2 {
  const float* part[BIAS_MAX];
  float* grad[BIAS_MAX];
  float* w[BIAS_MAX];
  float* v[BIAS_MAX];
  void* wb[BIAS_MAX];
  int nb[BIAS_MAX], C[BIAS_MAX];
  int gstart[BIAS_MAX + 1];   // first workgroup of each layer (32 bias elements per workgroup)
  int n;
  float lr, mom, wdlr;
  const float* rowloss;       // optional: loss = mean of rowloss[0..nrow), by one more workgroup
  int nrow;
  float* loss;
};
constexpr int BIAS_COLS = 32, BIAS_RG = TPB / BIAS_COLS;

template <typename T>
__global__ void __launch_bounds__(TPB) k_bias_colsum(BiasArgs1 a) {
  const int bid = blockIdx.x;
  int j = 0;
#pragma unroll
  for (int q = 1; q < BIAS_MAX; ++q) j += (q < a.n && bid >= a.bstart[q]) ? 1 : 0;
  const int local = bid - a.bstart[j];
  const int ctile = local / a.nb[j], rowblock = local - ctile * a.nb[j];
  if (a.f32[j])
    colsum_block<float>(static_cast<const float*>(a.x[j]), a.rows[j], a.C[j], a.rb[j], rowblock, ctile, a.part[j]);
  else
    colsum_block<T>(static_cast<const T*>(a.x[j]), a.rows[j], a.C[j], a.rb[j], rowblock, ctile, a.part[j]);
}

template <typename T>
__global__ void __launch_bounds__(TPB) k_bias_sgd(BiasArgs2 a) {
  const int bid = blockIdx.x, t = threadIdx.x;
  if (bid == a.gstart[a.n]) {
    // the batch-mean loss, by the first wave of the last workgroup
    if (!a.rowloss || t >= 64) return;
    float s = 0.f;
    for (int r = t; r < a.nrow; r += 64) s += a.rowloss[r];
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) s += __shfl_xor(s, o, 64);
    if (t == 0) *a.loss = s / (float)a.nrow;
    return;
  }
  int j = 0;
#pragma unroll
  for (int q = 1; q < BIAS_MAX; ++q) j += (q < a.n && bid >= a.gstart[q]) ? 1 : 0;
  const int C = a.C[j], nb = a.nb[j];
  const int cl = t % BIAS_COLS, rg = t / BIAS_COLS;
  const int col = (bid - a.gstart[j]) * BIAS_COLS + cl;
  const bool on = col < C;
  const float* part = a.part[j] + (on ? col : 0);
  float s = 0.f;
  int b = rg;
  for (; b + 7 * BIAS_RG < nb; b += 8 * BIAS_RG) {
    float q[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) q[u] = part[(int64_t)(b + u * BIAS_RG) * C];
#pragma unroll
    for (int u = 0; u < 8; ++u) s += q[u];
  }
  for (; b < nb; b += BIAS_RG) s += part[(int64_t)b * C];
  __shared__ float sh[BIAS_RG][BIAS_COLS];
  sh[rg][cl] = s;
  __syncthreads();
  if (rg == 0 && on) {
    float g = 0.f;
#pragma unroll
    for (int r = 0; r < BIAS_RG; ++r) g += sh[r][cl];
    a.grad[j][col] = g;
    float w = a.w[j][col], v = a.v[j][col];
    sgd_elem(w, v, g, a.mom, a.wdlr, a.lr);
    a.w[j][col] = w;
    a.v[j][col] = v;
    if (sizeof(T) == 2) static_cast<bf16*>(a.wb[j])[col] = f2bf(w);
    else static_cast<float*>(a.wb[j])[col] = w;
  }
}

size_t bias_grad_scratch_bytes(const BiasJob* jobs, int n) {
  size_t b = 0;
  for (int j = 0; j < n; ++j) b += (size_t)colsum_blocks(jobs[j].rows, jobs[j].C) * jobs[j].C * sizeof(float);
  return b;
}

hipError_t bias_grads_sgd(DType dt, const BiasJob* jobs, int n, const SgdHyper& hy, float* scratch,
                          const float* rowloss, int nrow, float* loss, hipStream_t st, const KTimer* kt) {
  if (n < 1 || n > BIAS_MAX) return hipErrorInvalidValue;
  BiasArgs1 a1 = {};
  BiasArgs2 a2 = {};
  a2.rowloss = rowloss;
  a2.nrow = nrow;
  a2.loss = loss;
  a1.n = a2.n = n;
  int blocks = 0, groups = 0;
  float* part = scratch;
  for (int j = 0; j < n; ++j) {
    const BiasJob& b = jobs[j];
    if (b.C % 8 || b.rows < 1) return hipErrorInvalidValue;
    const int nb = colsum_blocks(b.rows, b.C);
    a1.x[j] = b.dy;
    a1.part[j] = part;
    a1.rows[j] = b.rows;
    a1.rb[j] = (b.rows + nb - 1) / nb;
    a1.C[j] = b.C;
    a1.nb[j] = nb;
    a1.f32[j] = b.f32 ? 1 : 0;
    a1.bstart[j] = blocks;
    blocks += nb * cdiv(b.C, COLSUM_CW);
    a2.part[j] = part;
    a2.grad[j] = b.grad;
    a2.w[j] = b.w;
    a2.v[j] = b.v;
    a2.wb[j] = b.wb;
    a2.nb[j] = nb;
    a2.C[j] = b.C;
    a2.gstart[j] = groups;
    groups += cdiv(b.C, BIAS_COLS);
    part += (size_t)nb * b.C;
  }
  a1.bstart[n] = blocks;
  a2.gstart[n] = groups;
  a2.lr = hy.lr;
  a2.mom = hy.mom;
  a2.wdlr = hy.wdlr;
  rec_start(kt, st);
  if (dt == BF16) {
    hipLaunchKernelGGL((k_bias_colsum<bf16>), dim3(blocks), dim3(TPB), 0, st, a1);
    hipLaunchKernelGGL((k_bias_sgd<bf16>), dim3(groups + 1), dim3(TPB), 0, st, a2);
  } else {
    hipLaunchKernelGGL((k_bias_colsum<float>), dim3(blocks), dim3(TPB), 0, st, a1);
    hipLaunchKernelGGL((k_bias_sgd<float>), dim3(groups + 1), dim3(TPB), 0, st, a2);
  }
  rec_stop(kt, st);
  return hipGetLastError();
}

// =========================================================================
// Working copies of all 16 parameter tensors from their fp32 masters (round
// to nearest even for bf16), one launch.  Four elements per thread.
// =========================================================================
struct CastArgs {
  const float* w[16];
  void* wb[16];
  int64_t start[17];   // first 4-element chunk of each tensor
};

__device__ __forceinline__ int find_tensor(const int64_t* start, int64_t c) {
  int ti = 0;
#pragma unroll
  for (int i = 1; i < 16; ++i) ti += c >= start[i] ? 1 : 0;
  return ti;
}

template <typename T>
__global__ void k_cast_weights(CastArgs a) {
  const int64_t c = (int64_t)blockIdx.x * TPB + threadIdx.x;
  if (c >= a.start[16]) return;
  const int ti = find_tensor(a.start, c);
  const int64_t e = (c - a.start[ti]) * 4;
  const float4 w = *reinterpret_cast<const float4*>(a.w[ti] + e);
  T* o = reinterpret_cast<T*>(a.wb[ti]) + e;
  if (sizeof(T) == 2) {
    const uint32_t lo = f2bf2(w.x, w.y);
    const uint32_t hi = f2bf2(w.z, w.w);
    *reinterpret_cast<uint2*>(o) = make_uint2(lo, hi);
  } else {
    *reinterpret_cast<float4*>(o) = w;
  }
}

hipError_t cast_weights(DType dt, const TensorSet& ts, hipStream_t st) {
  CastArgs a;
  a.start[0] = 0;
  for (int i = 0; i < 16; ++i) {
    if (ts.n[i] % 4) return hipErrorInvalidValue;
    a.w[i] = ts.master[i]; a.wb[i] = ts.work[i];
    a.start[i + 1] = a.start[i] + ts.n[i] / 4;
  }
  const dim3 g = grid1d(a.start[16]);
  if (dt == BF16) hipLaunchKernelGGL((k_cast_weights<bf16>), g, dim3(TPB), 0, st, a);
  else hipLaunchKernelGGL((k_cast_weights<float>), g, dim3(TPB), 0, st, a);
  return hipGetLastError();
}

// =========================================================================
// Dropout keep-mask (the same draw the FC6/FC7 epilogues make)
// =========================================================================
__global__ void k_dropout_mask(uint64_t seed, uint64_t step, int layer, int64_t total, uint32_t thresh,
                               uint8_t* __restrict__ mask) {
  const int64_t q = (int64_t)blockIdx.x * TPB + threadIdx.x;
  if (q * 4 >= total) return;
  const uint4 r = philox4x32_10(make_uint4((uint32_t)q, (uint32_t)layer, (uint32_t)step, (uint32_t)(step >> 32)),
                                (uint32_t)seed, (uint32_t)(seed >> 32));
  const uint32_t w = (r.x < thresh ? 0u : 1u) | ((r.y < thresh ? 0u : 1u) << 8) |
                     ((r.z < thresh ? 0u : 1u) << 16) | ((r.w < thresh ? 0u : 1u) << 24);
  *reinterpret_cast<uint32_t*>(mask + q * 4) = w;
}
hipError_t dropout_mask(uint64_t seed, uint64_t step, int layer, int rows, int cols, uint32_t thresh,
                        uint8_t* mask, hipStream_t st) {
  const int64_t total = (int64_t)rows * cols;
  hipLaunchKernelGGL(k_dropout_mask, grid1d(total / 4), dim3(TPB), 0, st, seed, step, layer, total, thresh,
                     mask);
  return hipGetLastError();
}

}  // namespace ax
