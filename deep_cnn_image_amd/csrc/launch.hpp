// Host-side launchers for the AlexNet HIP kernels.  Every launcher enqueues on
// `st` and returns the launch status; shapes are checked by the caller.
#pragma once
#include <hip/hip_runtime_api.h>
#include <stddef.h>
#include <stdint.h>

namespace ax {

enum DType { F32 = 0, BF16 = 1 };

// Optional events recorded on the launch stream right before and after one
// kernel launch (the MFMA kernel for GEMM layers).
struct KTimer {
  hipEvent_t start, stop;
};

inline int cdiv(int64_t a, int64_t b) { return (int)((a + b - 1) / b); }

// Reduction depth of one GEMM k-tile (elements).
constexpr int GEMM_BK = 64;

// Split-K factor actually used for K (in elements) when `want` splits are
// requested: every split gets at least one k-tile and none is empty.
inline int eff_splits(int K, int want) {
  const int kt = cdiv(K, GEMM_BK);
  if (want < 1) want = 1;
  if (want > kt) want = kt;
  const int per = cdiv(kt, want);
  return cdiv(kt, per);
}

struct ConvShape {
  int Nimg, H, W, Cin, Cout, K, stride, pad, groups, Ho, Wo;
};

// ---- weight re-layouts (per call; weights change every training step), all
// in one launch.  src is an OIHW tensor of Cout x Cig x K x K (Cig = input
// channels per group), G the group count.
enum { WPREP_W1S = 0, WPREP_KHWC = 1, WPREP_DGRAD = 2 };
constexpr int WPREP_MAX = 9;
struct WeightPrep {
  int kind;
  const void* src;
  void* dst;
  int Cout, Cig, K, G;
};
// Training-time augmentation of a batch of Hs x Ws sources (device arrays):
// image n is the 227 x 227 patch of source n at (y0, x0) = crop[n][0..1]
// (clamped into the source), mirrored left-right if crop[n][2] != 0, plus the
// RGB shift sum_i eigvec[c][i] * alpha[n][i] * eigval[i] on channel c.
struct AugSrc {
  const int32_t* crop;   // [N][3]
  const float* alpha;    // [N][3]
  const float* eigvec;   // [3][3], column i = component i
  const float* eigval;   // [3]
};
// Layer-1 input sources: 227 x 227 images, ten-view crops of 256 x 256
// sources, or augmented patches of Hs x Ws sources.
enum { SRC_IMAGES = 0, SRC_TENVIEW = 1, SRC_AUGMENT = 2 };
// One launch: the weight re-layouts `jobs` and the layer-1 input staging
// (xs from the NCHW images x, the ten-view crops or the augmented patches;
// `aug` is read only for SRC_AUGMENT).
hipError_t stage_inputs(DType, const WeightPrep* jobs, int n, const void* x, int Hs, int Ws, int src_kind,
                        const AugSrc* aug, int Nimg, void* xs, hipStream_t, const KTimer* kt = nullptr);
// x_out [N][3][227][227] = the augmented patches (same values stage_inputs
// stages for SRC_AUGMENT).
hipError_t augment_images(DType, const void* src, int Hs, int Ws, const AugSrc& aug, int Nimg, void* x_out,
                          hipStream_t);
// Principal components of the RGB values of every pixel of n images
// [n][3][H][W]: covariance (divided by the pixel count) accumulated in fp64,
// eigen-decomposed by cyclic Jacobi rotations; eigval [3] descending, eigvec
// [3][3] with column i the unit eigenvector of eigval[i], signed so that its
// largest-magnitude entry is positive.  `scratch` holds rgb_pca_scratch_bytes().
size_t rgb_pca_scratch_bytes();
hipError_t rgb_pca(DType, const void* src, int n, int H, int W, float* eigval, float* eigvec, void* scratch,
                   hipStream_t, const KTimer* kt = nullptr);

// ---- convolutions (bf16 MFMA or fp32 MFMA, fp32 accumulate)
// Layer 1 runs as a 3x3 stride-1 convolution over 4x4 pixel blocks:
// xs [N][57][57][48] from NCHW images (or ten-view sources, cropped and
// mirrored), ws [96][432] from the OIHW weights.
constexpr size_t S2D_ELEMS = 57 * 57 * 48;   // per image
constexpr size_t S2D_W_ELEMS = 96 * 432;

// y NHWC [N][55][55][96] = relu(conv1 + b).  bf16: a direct convolution with
// the block rows in LDS (no partials); fp32: an implicit GEMM whose split-K
// partials go to part, at least conv1_fwd_part_bytes (0 unless the batch is
// too small to fill the chip).
hipError_t conv1_fwd(DType, const void* xs, int Nimg, const void* ws, const void* b1, void* y, float* part,
                     size_t part_bytes, hipStream_t, const KTimer* kt = nullptr);
// NHWC conv + bias + ReLU (layers 2-5); part as for conv1_fwd, at least
// conv_fwd_part_bytes.
hipError_t conv_fwd(DType, const ConvShape&, const void* x, const void* wr, const void* b, void* y, float* part,
                    size_t part_bytes, hipStream_t, const KTimer* kt = nullptr);
size_t conv1_fwd_part_bytes(DType, int Nimg);
size_t conv_fwd_part_bytes(DType, const ConvShape&);
// dX (NHWC) = conv^T(dY) * [mask > 0] (mask optional) for stride-1 layers;
// part as for conv1_fwd, at least conv_dgrad_part_bytes.
hipError_t conv_dgrad(DType, const ConvShape&, const void* dy, const void* wt, const void* mask,
                      void* dx, float* part, size_t part_bytes, hipStream_t, const KTimer* kt = nullptr);
size_t conv_dgrad_part_bytes(DType, const ConvShape&);
// SGD hyper-parameters: learning rate, momentum, weight decay times learning rate.
struct SgdHyper { float lr, mom, wdlr; };
// Optional SGD applied to a weight gradient as it is reduced: fp32 master w and
// momentum v (same layout as the gradient) in place, working copy wb in the
// compute type; w == nullptr: gradient only.
struct SgdTarget { float* w; float* v; void* wb; SgdHyper hy; };
// fp32 weight gradient (OIHW) of layers 2-5; `part` is split-K scratch
hipError_t conv_wgrad(DType, const ConvShape&, const void* dy, const void* x, float* part,
                      size_t part_bytes, float* gw, const SgdTarget* sgd, hipStream_t,
                      const KTimer* kt = nullptr);
// fp32 weight gradient (OIHW) of layer 1 from the space-to-depth input xs;
// part at least conv1_wgrad_part_bytes (bf16: one partial per workgroup of
// the direct kernel; fp32: split-K partials)
hipError_t conv1_wgrad(DType, int Nimg, const void* dy, const void* xs, float* part, size_t part_bytes,
                       float* gw, const SgdTarget* sgd, hipStream_t,
                      const KTimer* kt = nullptr);
size_t conv_wgrad_part_bytes(const ConvShape&);
size_t conv1_wgrad_part_bytes(DType, int Nimg);

// ---- fully-connected layers
struct FcEpi {
  int relu;             // 1: ReLU
  int drop;             // 0: none, 1: Philox keep-mask (training), 2: multiply by `scale`
  float scale;
  uint32_t thresh;      // drop iff Philox word < thresh
  uint64_t seed, step;
  int layer;
};
// y[M][O] = epi(x[M][K] W[O][K]^T + b); y is cfg dtype, or fp32 if y_f32
hipError_t fc_fwd(DType, int M, int K, int O, const void* x, const void* w, const void* b,
                  const FcEpi&, void* y, float* y_f32, float* part, size_t part_bytes, hipStream_t,
                      const KTimer* kt = nullptr);
// dx[M][K] = (dy[M][O] W[O][K]) * [mask > 0] (mask optional)
hipError_t fc_dgrad(DType, int M, int K, int O, const void* dy, const void* w, const void* mask,
                    void* dx, float* part, size_t part_bytes, hipStream_t,
                      const KTimer* kt = nullptr);
// dW[O][K] fp32 = dy^T x
// SGD hyper-parameters as the update uses them (wdlr = weight decay * lr).
// FC weight gradient dW = dY^T X, applied at once to the layer's fp32 master
// weights w, momentum v and working copy wb (sgd_elem); dW is not stored.
hipError_t fc_wgrad_sgd(DType, int M, int K, int O, const void* dy, const void* x, const SgdHyper& h,
                        float* w, float* v, void* wb, hipStream_t, const KTimer* kt = nullptr);
size_t fc_fwd_part_bytes(int M, int K, int O);
size_t fc_dgrad_part_bytes(int M, int K, int O);

// ---- bandwidth-bound layers (NHWC, C % 8 == 0)
// LRN then 3x3 / stride-2 max-pool with argmax in one pass over the input;
// `dbg` (may be null) also receives the LRN output.
hipError_t lrn_pool_fwd(DType, const void* a, void* y, uint8_t* arg, void* dbg, int N, int H, int W, int C,
                        float k, float alpha, float beta, int n, hipStream_t, const KTimer* kt = nullptr);
// Max-pool backward, LRN backward and the preceding ReLU's mask in one pass:
// dy (pooled gradient) and arg -> da w.r.t. the LRN input a.  `dbg` (may be
// null) also receives the gradient w.r.t. the LRN output.  `bias_rows` (may
// be null) receives, per row (n, h) of da, the column sums of its stored
// values, fp32 [N * H][C]: the layer's bias gradient summed over w.
hipError_t pool_lrn_bwd(DType, const void* dy, const uint8_t* arg, const void* a, void* da, void* dbg,
                        float* bias_rows, int N, int H, int W, int C, float k, float alpha, float beta, int n,
                        hipStream_t, const KTimer* kt = nullptr);
// 3x3/s2 max-pool; flat_out: y written [N][C*Ho*Wo] in (c,h,w) order
// Pool 5 (3x3 / stride 2) with its output flattened in (c, h, w) order for
// FC6, and its backward times the ReLU mask of the pool input.  C % 128 == 0.
hipError_t pool5_fwd(DType, const void* x, void* y_flat, uint8_t* arg, int N, int H, int W, int C, hipStream_t,
                     const KTimer* kt = nullptr);
hipError_t pool5_bwd(DType, const void* dy_flat, const uint8_t* arg, const void* mask, void* dx, int N, int H,
                     int W, int C, hipStream_t, const KTimer* kt = nullptr);

// ---- network head, ten-view mean, column sums
// FC8 and the softmax: logits[M][O] fp32 = x W^T + b (split-K GEMM), then
// p = softmax(logits) (p may be null); with labels also dz = (p - onehot)/M
// in the compute type and rowloss[m] = -log p[m][label].  O % 4 == 0, O <= 1024.
hipError_t fc_head(DType, int M, int K, int O, const void* x, const void* w, const void* b, float* logits,
                   const int32_t* labels, float* p, void* dz, float* rowloss, float* part, size_t part_bytes,
                   hipStream_t, const KTimer* kt = nullptr);
hipError_t view_mean(const float* p, float* out, int N, int O, hipStream_t);
// Bias gradients of up to BIAS_MAX layers, grad[c] = sum over the rows of
// dy[rows][C] (fp32), each followed by the SGD update of the bias (w, v fp32
// in place; wb the working copy in the compute type).  dy is in the compute
// type, or fp32 with `f32` (row partial sums left by the kernel that made the
// gradient).  Partial sums go to `scratch` (bias_grad_scratch_bytes).
constexpr int BIAS_MAX = 8;
struct BiasJob {
  const void* dy;
  int64_t rows;
  int C;
  float* grad;
  float* w;
  float* v;
  void* wb;
  bool f32;
};
size_t bias_grad_scratch_bytes(const BiasJob* jobs, int n);
// Also, if rowloss is not null, *loss = mean of rowloss[0..nrow) (fixed order).
hipError_t bias_grads_sgd(DType, const BiasJob* jobs, int n, const SgdHyper& hy, float* scratch,
                          const float* rowloss, int nrow, float* loss, hipStream_t, const KTimer* kt = nullptr);

// ---- working-copy cast, dropout mask
struct TensorSet {
  const float* master[16];
  void* work[16];
  int64_t n[16];
};
hipError_t cast_weights(DType work_dtype, const TensorSet&, hipStream_t);
hipError_t dropout_mask(uint64_t seed, uint64_t step, int layer, int rows, int cols,
                        uint32_t thresh, uint8_t* mask, hipStream_t);

}  // namespace ax
