/*
 * AlexNet CPU oracle -- TEST INFRASTRUCTURE ONLY.
 *
 * A plain, slow, direct-loop implementation of every operation on the AlexNet
 * forward and training-step path, written from the definitions on the pages
 * (Krizhevsky, Sutskever, Hinton, "ImageNet Classification with Deep
 * Convolutional Neural Networks", NeurIPS 2012, as summarised on the
 * paper-graph-ui page, the bloss0m.com reading notes and the fermi.ai wiki).
 *
 * Only the test suite, the smoke check and the CPU-baseline leg of the
 * benchmark may load this library.  It shares no code, header, table or
 * helper with the HIP library; it never calls into it and is never called by it.
 *
 * Conventions
 *  - Tensors are NCHW (conv) / [rows][features] (FC), dense, row-major.
 *  - Every value is double.  Sums accumulate in double, in the order the loops
 *    state; there is no blocking, fusion or reordering of the arithmetic beyond
 *    choosing which loop runs innermost.
 *  - OpenMP parallelises over independent outputs only (each thread owns the
 *    outputs it writes), so results do not depend on the thread count.
 *
 * Parity status of each function is given in its comment; the pins live in
 * tests/test_oracle_*.py.
 */
#include <cmath>
#include <cstdint>
#include <cstring>
#include <vector>
#ifdef _OPENMP
#include <omp.h>
#endif

extern "C" {

/* ------------------------------------------------------------------------ *
 * Convolution, forward.
 * Pages: paper-graph-ui "Overall Architecture (Layer-by-Layer Specification)"
 * (kernel counts, sizes, stride 4 on layer 1, the same-GPU connectivity of
 * layers 2, 4, 5) and the fermi.ai layer list (paddings 0/2/1/1/1).
 *
 *   y[n,co,h,w] = b[co] + sum_{ci'<Cin/G} sum_{kh,kw}
 *                 W[co,ci',kh,kw] * x[n, g*Cin/G + ci', h*s-p+kh, w*s-p+kw]
 *   with g = co / (Cout/G) and x taken as zero outside the image.
 * Pinned by: torch float64 conv2d, delta-kernel and constant-input closed forms.
 * ------------------------------------------------------------------------ */
void orc_conv2d_fwd(const double* x, int N, int Cin, int H, int W,
                    const double* w, const double* b, int Cout, int K, int stride,
                    int pad, int G, double* y) {
  const int Ho = (H + 2 * pad - K) / stride + 1;
  const int Wo = (W + 2 * pad - K) / stride + 1;
  const int cin_g = Cin / G, cout_g = Cout / G;
#pragma omp parallel for collapse(2) schedule(dynamic)
  for (int n = 0; n < N; ++n)
    for (int co = 0; co < Cout; ++co) {
      const int g = co / cout_g;
      double* out = y + ((size_t)n * Cout + co) * Ho * Wo;
      for (int i = 0; i < Ho * Wo; ++i) out[i] = b ? b[co] : 0.0;
      for (int cl = 0; cl < cin_g; ++cl) {
        const int ci = g * cin_g + cl;
        const double* in = x + ((size_t)n * Cin + ci) * H * W;
        for (int kh = 0; kh < K; ++kh)
          for (int kw = 0; kw < K; ++kw) {
            const double wv = w[(((size_t)co * cin_g + cl) * K + kh) * K + kw];
            for (int ho = 0; ho < Ho; ++ho) {
              const int hi = ho * stride - pad + kh;
              if (hi < 0 || hi >= H) continue;
              for (int wo = 0; wo < Wo; ++wo) {
                const int wi = wo * stride - pad + kw;
                if (wi < 0 || wi >= W) continue;
                out[ho * Wo + wo] += wv * in[hi * W + wi];
              }
            }
          }
      }
    }
}

/* Convolution, gradient w.r.t. the input: the transpose of the index map of
 * orc_conv2d_fwd (backpropagation of the pages' training procedure).
 *   dx[n,ci,hi,wi] = sum over (co in ci's group, kh, kw, ho, wo) with
 *                    ho*s-p+kh == hi and wo*s-p+kw == wi of W[co,ci',kh,kw]*dy[n,co,ho,wo]
 * Each thread owns one (n, ci) plane of dx.
 * Pinned by: torch float64 autograd of conv2d; central differences.        */
void orc_conv2d_bwd_data(const double* dy, int N, int Cin, int H, int W,
                         const double* w, int Cout, int K, int stride, int pad, int G,
                         double* dx) {
  const int Ho = (H + 2 * pad - K) / stride + 1;
  const int Wo = (W + 2 * pad - K) / stride + 1;
  const int cin_g = Cin / G, cout_g = Cout / G;
#pragma omp parallel for collapse(2) schedule(dynamic)
  for (int n = 0; n < N; ++n)
    for (int ci = 0; ci < Cin; ++ci) {
      const int g = ci / cin_g, cl = ci % cin_g;
      double* out = dx + ((size_t)n * Cin + ci) * H * W;
      for (int i = 0; i < H * W; ++i) out[i] = 0.0;
      for (int col = 0; col < cout_g; ++col) {
        const int co = g * cout_g + col;
        const double* gy = dy + ((size_t)n * Cout + co) * Ho * Wo;
        for (int kh = 0; kh < K; ++kh)
          for (int kw = 0; kw < K; ++kw) {
            const double wv = w[(((size_t)co * cin_g + cl) * K + kh) * K + kw];
            for (int ho = 0; ho < Ho; ++ho) {
              const int hi = ho * stride - pad + kh;
              if (hi < 0 || hi >= H) continue;
              for (int wo = 0; wo < Wo; ++wo) {
                const int wi = wo * stride - pad + kw;
                if (wi < 0 || wi >= W) continue;
                out[hi * W + wi] += wv * gy[ho * Wo + wo];
              }
            }
          }
      }
    }
}

/* Convolution, gradient w.r.t. weights and bias.
 *   dW[co,ci',kh,kw] = sum_{n,ho,wo} dy[n,co,ho,wo] * x[n, g*Cin/G+ci', ho*s-p+kh, wo*s-p+kw]
 *   db[co]           = sum_{n,ho,wo} dy[n,co,ho,wo]
 * Pinned by: torch float64 autograd; central differences.                 */
void orc_conv2d_bwd_weight(const double* dy, const double* x, int N, int Cin, int H,
                           int W, int Cout, int K, int stride, int pad, int G,
                           double* dw, double* db) {
  const int Ho = (H + 2 * pad - K) / stride + 1;
  const int Wo = (W + 2 * pad - K) / stride + 1;
  const int cin_g = Cin / G, cout_g = Cout / G;
#pragma omp parallel for collapse(2) schedule(dynamic)
  for (int co = 0; co < Cout; ++co)
    for (int cl = 0; cl < cin_g; ++cl) {
      const int g = co / cout_g, ci = g * cin_g + cl;
      for (int kh = 0; kh < K; ++kh)
        for (int kw = 0; kw < K; ++kw) {
          double acc = 0.0;
          for (int n = 0; n < N; ++n) {
            const double* gy = dy + ((size_t)n * Cout + co) * Ho * Wo;
            const double* in = x + ((size_t)n * Cin + ci) * H * W;
            for (int ho = 0; ho < Ho; ++ho) {
              const int hi = ho * stride - pad + kh;
              if (hi < 0 || hi >= H) continue;
              for (int wo = 0; wo < Wo; ++wo) {
                const int wi = wo * stride - pad + kw;
                if (wi < 0 || wi >= W) continue;
                acc += gy[ho * Wo + wo] * in[hi * W + wi];
              }
            }
          }
          dw[(((size_t)co * cin_g + cl) * K + kh) * K + kw] = acc;
        }
    }
  if (db) {
#pragma omp parallel for
    for (int co = 0; co < Cout; ++co) {
      double acc = 0.0;
      for (int n = 0; n < N; ++n) {
        const double* gy = dy + ((size_t)n * Cout + co) * Ho * Wo;
        for (int i = 0; i < Ho * Wo; ++i) acc += gy[i];
      }
      db[co] = acc;
    }
  }
}

/* ------------------------------------------------------------------------ *
 * ReLU: f(x) = max(0, x)  (paper-graph-ui "ReLU Nonlinearity").
 * Backward: derivative 1 for x > 0 and 0 otherwise; the subgradient at 0 is
 * taken as 0.  Given the ReLU *output* a, the mask is [a > 0].
 * Pinned by: invariants (out >= 0, identity on positives).
 * ------------------------------------------------------------------------ */
void orc_relu(const double* x, int64_t n, double* y) {
#pragma omp parallel for
  for (int64_t i = 0; i < n; ++i) y[i] = x[i] > 0.0 ? x[i] : 0.0;
}
void orc_relu_bwd(const double* a, const double* g, int64_t n, double* gz) {
#pragma omp parallel for
  for (int64_t i = 0; i < n; ++i) gz[i] = a[i] > 0.0 ? g[i] : 0.0;
}

/* ------------------------------------------------------------------------ *
 * Local response normalisation (paper-graph-ui "Local Response
 * Normalization", the displayed equation and its constants):
 *   b_i = a_i / (k + alpha * sum_{j=max(0,i-n/2)}^{min(N-1,i+n/2)} a_j^2)^beta
 * over the channel axis at one (n, y, x); n/2 is the integer half-width
 * (n = 5 -> 2); N = all channels of the layer.  alpha multiplies the sum
 * directly (it is not divided by n).
 * Pinned by: torch float64 local_response_norm with alpha*n, closed forms for
 * zero, single-channel and constant inputs.
 * ------------------------------------------------------------------------ */
void orc_lrn_fwd(const double* a, int N, int C, int HW, double k, double alpha,
                 double beta, int nsize, double* b) {
  const int half = nsize / 2;
#pragma omp parallel for collapse(2)
  for (int n = 0; n < N; ++n)
    for (int p = 0; p < HW; ++p) {
      const double* an = a + (size_t)n * C * HW;
      double* bn = b + (size_t)n * C * HW;
      for (int i = 0; i < C; ++i) {
        const int lo = i - half < 0 ? 0 : i - half;
        const int hi = i + half > C - 1 ? C - 1 : i + half;
        double s = 0.0;
        for (int j = lo; j <= hi; ++j) s += an[(size_t)j * HW + p] * an[(size_t)j * HW + p];
        bn[(size_t)i * HW + p] = an[(size_t)i * HW + p] / std::pow(k + alpha * s, beta);
      }
    }
}

/* LRN backward, the derivative of orc_lrn_fwd.  With
 *   S_i = k + alpha * sum_{j in W(i)} a_j^2,  b_i = a_i * S_i^-beta,
 *   db_i/da_j = [i==j] S_i^-beta - 2 alpha beta a_i a_j S_i^(-beta-1) [j in W(i)],
 * and since j in W(i) <=> |i-j| <= n/2 (both in range), the window is symmetric:
 *   da_j = g_j S_j^-beta - 2 alpha beta a_j sum_{i in W(j)} g_i a_i S_i^(-beta-1).
 * Pinned by: torch float64 autograd of local_response_norm; central differences. */
void orc_lrn_bwd(const double* a, const double* g, int N, int C, int HW, double k,
                 double alpha, double beta, int nsize, double* da) {
  const int half = nsize / 2;
#pragma omp parallel for collapse(2)
  for (int n = 0; n < N; ++n)
    for (int p = 0; p < HW; ++p) {
      const double* an = a + (size_t)n * C * HW;
      const double* gn = g + (size_t)n * C * HW;
      double* dn = da + (size_t)n * C * HW;
      std::vector<double> S(C);
      for (int i = 0; i < C; ++i) {
        const int lo = i - half < 0 ? 0 : i - half;
        const int hi = i + half > C - 1 ? C - 1 : i + half;
        double s = 0.0;
        for (int j = lo; j <= hi; ++j) s += an[(size_t)j * HW + p] * an[(size_t)j * HW + p];
        S[i] = k + alpha * s;
      }
      for (int j = 0; j < C; ++j) {
        const int lo = j - half < 0 ? 0 : j - half;
        const int hi = j + half > C - 1 ? C - 1 : j + half;
        double cross = 0.0;
        for (int i = lo; i <= hi; ++i)
          cross += gn[(size_t)i * HW + p] * an[(size_t)i * HW + p] * std::pow(S[i], -beta - 1.0);
        dn[(size_t)j * HW + p] = gn[(size_t)j * HW + p] * std::pow(S[j], -beta) -
                                 2.0 * alpha * beta * an[(size_t)j * HW + p] * cross;
      }
    }
}

/* ------------------------------------------------------------------------ *
 * Overlapping max-pooling (paper-graph-ui "Overlapping Pooling": z = 3,
 * s = 2).  out[n,c,i,j] = max_{dy,dx<z} in[n,c,s*i+dy,s*j+dx], output size
 * (H-z)/s+1.  argmax is the first maximum of a row-major scan of the window
 * (replace only on strictly greater), stored as dy*z+dx in one byte.
 * Pinned by: torch float64 max_pool2d values/indices on tie-free inputs,
 * invariants, constant-plane tie rule.
 * ------------------------------------------------------------------------ */
void orc_maxpool_fwd(const double* x, int N, int C, int H, int W, int z, int s,
                     double* y, uint8_t* arg) {
  const int Ho = (H - z) / s + 1, Wo = (W - z) / s + 1;
#pragma omp parallel for collapse(2)
  for (int n = 0; n < N; ++n)
    for (int c = 0; c < C; ++c) {
      const double* in = x + ((size_t)n * C + c) * H * W;
      double* out = y + ((size_t)n * C + c) * Ho * Wo;
      uint8_t* am = arg + ((size_t)n * C + c) * Ho * Wo;
      for (int i = 0; i < Ho; ++i)
        for (int j = 0; j < Wo; ++j) {
          double best = in[(s * i) * W + s * j];
          int bi = 0;
          for (int dy = 0; dy < z; ++dy)
            for (int dx = 0; dx < z; ++dx) {
              const double v = in[(s * i + dy) * W + s * j + dx];
              if (v > best) { best = v; bi = dy * z + dx; }
            }
          out[i * Wo + j] = best;
          am[i * Wo + j] = (uint8_t)bi;
        }
    }
}

/* Max-pool backward: every output gradient goes to the input position its
 * argmax names; positions named by several overlapping windows receive the
 * sum.  Each thread owns one (n, c) plane.                                    */
void orc_maxpool_bwd(const double* dy, const uint8_t* arg, int N, int C, int H, int W,
                     int z, int s, double* dx) {
  const int Ho = (H - z) / s + 1, Wo = (W - z) / s + 1;
#pragma omp parallel for collapse(2)
  for (int n = 0; n < N; ++n)
    for (int c = 0; c < C; ++c) {
      double* out = dx + ((size_t)n * C + c) * H * W;
      const double* g = dy + ((size_t)n * C + c) * Ho * Wo;
      const uint8_t* am = arg + ((size_t)n * C + c) * Ho * Wo;
      for (int i = 0; i < H * W; ++i) out[i] = 0.0;
      for (int i = 0; i < Ho; ++i)
        for (int j = 0; j < Wo; ++j) {
          const int dyy = am[i * Wo + j] / z, dxx = am[i * Wo + j] % z;
          out[(s * i + dyy) * W + s * j + dxx] += g[i * Wo + j];
        }
    }
}

/* ------------------------------------------------------------------------ *
 * Fully-connected layer (paper-graph-ui "Overall Architecture", layers 6-8):
 *   y[m,o] = b[o] + sum_k W[o,k] x[m,k],  W stored [out][in].
 * Backward: dx[m,k] = sum_o dy[m,o] W[o,k]; dW[o,k] = sum_m dy[m,o] x[m,k];
 *           db[o] = sum_m dy[m,o].
 * Pinned by: torch float64 linear and autograd.
 * ------------------------------------------------------------------------ */
void orc_fc_fwd(const double* x, int M, int K, const double* w, const double* b, int O,
                double* y) {
#pragma omp parallel for collapse(2)
  for (int m = 0; m < M; ++m)
    for (int o = 0; o < O; ++o) {
      double acc = b ? b[o] : 0.0;
      const double* xr = x + (size_t)m * K;
      const double* wr = w + (size_t)o * K;
      for (int k = 0; k < K; ++k) acc += wr[k] * xr[k];
      y[(size_t)m * O + o] = acc;
    }
}

void orc_fc_bwd(const double* dy, const double* x, const double* w, int M, int K, int O,
                double* dx, double* dw, double* db) {
  // Each output element is a sum over o (for dx) or m (for dW) taken in
  // ascending order; the loops run along rows so W and x are read contiguously.
  if (dx) {
#pragma omp parallel for
    for (int m = 0; m < M; ++m) {
      double* out = dx + (size_t)m * K;
      for (int k = 0; k < K; ++k) out[k] = 0.0;
      for (int o = 0; o < O; ++o) {
        const double d = dy[(size_t)m * O + o];
        const double* wr = w + (size_t)o * K;
        for (int k = 0; k < K; ++k) out[k] += d * wr[k];
      }
    }
  }
#pragma omp parallel for
  for (int o = 0; o < O; ++o) {
    double* out = dw + (size_t)o * K;
    for (int k = 0; k < K; ++k) out[k] = 0.0;
    for (int m = 0; m < M; ++m) {
      const double d = dy[(size_t)m * O + o];
      const double* xr = x + (size_t)m * K;
      for (int k = 0; k < K; ++k) out[k] += d * xr[k];
    }
    if (db) {
      double acc = 0.0;
      for (int m = 0; m < M; ++m) acc += dy[(size_t)m * O + o];
      db[o] = acc;
    }
  }
}

/* ------------------------------------------------------------------------ *
 * Softmax over each row (the 1000-way output of layer 8):
 *   p_i = exp(z_i - max z) / sum_j exp(z_j - max z).
 * Pinned by: sum to 1, shift invariance, the husky/Eskimo-dog logit pair on
 * the fermi.ai page (ratio e^0.8), torch float64 softmax.
 * ------------------------------------------------------------------------ */
void orc_softmax(const double* z, int M, int O, double* p) {
#pragma omp parallel for
  for (int m = 0; m < M; ++m) {
    const double* zr = z + (size_t)m * O;
    double* pr = p + (size_t)m * O;
    double mx = zr[0];
    for (int i = 1; i < O; ++i) mx = zr[i] > mx ? zr[i] : mx;
    double s = 0.0;
    for (int i = 0; i < O; ++i) { pr[i] = std::exp(zr[i] - mx); s += pr[i]; }
    for (int i = 0; i < O; ++i) pr[i] /= s;
  }
}

/* Multinomial logistic regression objective (paper-graph-ui "Training
 * Procedure Details", objective function): the mean over the batch of the
 * negative log-probability of the correct label, and its gradient w.r.t. the
 * logits, (p - onehot(y)) / M.
 * Pinned by: torch float64 cross_entropy and its autograd.                  */
double orc_ce_loss_grad(const double* p, const int32_t* labels, int M, int O, double* dz) {
  double loss = 0.0;
  for (int m = 0; m < M; ++m) loss -= std::log(p[(size_t)m * O + labels[m]]);
  loss /= M;
  if (dz) {
    for (int m = 0; m < M; ++m)
      for (int i = 0; i < O; ++i)
        dz[(size_t)m * O + i] = (p[(size_t)m * O + i] - (i == labels[m] ? 1.0 : 0.0)) / M;
  }
  return loss;
}

/* ------------------------------------------------------------------------ *
 * SGD with momentum and weight decay (paper-graph-ui "Training Procedure
 * Details", the update-rule equations; fermi.ai TRAIN_STEP):
 *   v <- mu*v - lambda*eps*w - eps*g ;  w <- w + v
 * Pinned by: closed forms (g = 0, w = 0, a two-step recurrence by hand).
 * ------------------------------------------------------------------------ */
void orc_sgd(double* w, double* v, const double* g, int64_t n, double eps, double mu,
             double lambda) {
#pragma omp parallel for
  for (int64_t i = 0; i < n; ++i) {
    v[i] = mu * v[i] - lambda * eps * w[i] - eps * g[i];
    w[i] = w[i] + v[i];
  }
}

/* ------------------------------------------------------------------------ *
 * Philox4x32-10, from its published definition (Salmon, Moraes, Dror, Shaw,
 * "Parallel Random Numbers: As Easy as 1, 2, 3", SC'11): ten rounds of
 *   (hi0,lo0) = mulhilo(0xD2511F53, c0); (hi1,lo1) = mulhilo(0xCD9E8D57, c2)
 *   c <- (hi1 ^ c1 ^ k0, lo1, hi0 ^ c3 ^ k1, lo0)
 * with the key bumped by (0x9E3779B9, 0xBB67AE85) between rounds.
 * The pages only ask for dropout with probability 0.5; the counter-based
 * generator is how the masks are made reproducible.  Pinned word for word
 * against PyTorch's independent source-level engine (ATen PhiloxRNGEngine.h)
 * by tests/test_oracle_philox.py, and the mask statistics by
 * tests/test_oracle_layers.py.
 * ------------------------------------------------------------------------ */
static inline void orc_mulhilo(uint32_t a, uint32_t b, uint32_t* hi, uint32_t* lo) {
  const uint64_t p = (uint64_t)a * (uint64_t)b;
  *hi = (uint32_t)(p >> 32);
  *lo = (uint32_t)p;
}

void orc_philox4x32_10(const uint32_t ctr_in[4], const uint32_t key_in[2], uint32_t out[4]) {
  uint32_t c0 = ctr_in[0], c1 = ctr_in[1], c2 = ctr_in[2], c3 = ctr_in[3];
  uint32_t k0 = key_in[0], k1 = key_in[1];
  for (int r = 0; r < 10; ++r) {
    if (r > 0) { k0 += 0x9E3779B9u; k1 += 0xBB67AE85u; }
    uint32_t hi0, lo0, hi1, lo1;
    orc_mulhilo(0xD2511F53u, c0, &hi0, &lo0);
    orc_mulhilo(0xCD9E8D57u, c2, &hi1, &lo1);
    const uint32_t n0 = hi1 ^ c1 ^ k0, n1 = lo1, n2 = hi0 ^ c3 ^ k1, n3 = lo0;
    c0 = n0; c1 = n1; c2 = n2; c3 = n3;
  }
  out[0] = c0; out[1] = c1; out[2] = c2; out[3] = c3;
}

/* Dropout keep-mask for one fully-connected layer (paper-graph-ui "Dropout":
 * each hidden unit's output is zeroed with probability p during training).
 * Element e = row*cols + col of layer `layer` (0 = FC6, 1 = FC7) at training
 * step `step` draws word (e mod 4) of Philox4x32-10 with
 *   counter = (e / 4, layer, step mod 2^32, step / 2^32),
 *   key     = (seed mod 2^32, seed / 2^32),
 * and is dropped iff that word is below floor(p * 2^32).
 * mask[e] = 1 keeps the unit, 0 drops it.                                  */
void orc_dropout_mask(uint64_t seed, uint64_t step, int layer, int rows, int cols, double p,
                      uint8_t* mask) {
  const uint32_t thresh = (uint32_t)std::floor(p * 4294967296.0);
  const uint32_t key[2] = {(uint32_t)seed, (uint32_t)(seed >> 32)};
  const int64_t total = (int64_t)rows * cols;
#pragma omp parallel for
  for (int64_t q = 0; q < (total + 3) / 4; ++q) {
    const uint32_t ctr[4] = {(uint32_t)q, (uint32_t)layer, (uint32_t)step,
                             (uint32_t)(step >> 32)};
    uint32_t r[4];
    orc_philox4x32_10(ctr, key, r);
    for (int t = 0; t < 4; ++t) {
      const int64_t e = q * 4 + t;
      if (e < total) mask[e] = r[t] < thresh ? 0 : 1;
    }
  }
}

/* ------------------------------------------------------------------------ *
 * Ten-patch test-time views (paper-graph-ui "Data Augmentation", test-time
 * procedure): the four corner patches and the centre patch of each source
 * image, plus their horizontal reflections.  For a source of side S and a
 * crop of side P, offsets (y0,x0) are (0,0), (0,S-P), (S-P,0), (S-P,S-P),
 * ((S-P)/2,(S-P)/2) with integer halving; view v in [5,10) is view v-5
 * mirrored (x -> P-1-x).  Output index n*10 + v.
 * Pinned by: coordinate-encoding closed form, constant-image invariance.
 * ------------------------------------------------------------------------ */
void orc_tenview_crop(const double* src, int N, int C, int S, int P, double* out) {
  const int d = S - P;
  const int oy[5] = {0, 0, d, d, d / 2};
  const int ox[5] = {0, d, 0, d, d / 2};
#pragma omp parallel for collapse(2)
  for (int n = 0; n < N; ++n)
    for (int v = 0; v < 10; ++v) {
      const int base = v % 5;
      const bool flip = v >= 5;
      for (int c = 0; c < C; ++c)
        for (int y = 0; y < P; ++y)
          for (int x = 0; x < P; ++x) {
            const int sx = flip ? (P - 1 - x) : x;
            out[((((size_t)n * 10 + v) * C + c) * P + y) * P + x] =
                src[(((size_t)n * C + c) * S + oy[base] + y) * S + ox[base] + sx];
          }
    }
}

/* ------------------------------------------------------------------------ *
 * Training-time augmentation (paper-graph-ui "Data Augmentation", Form 1:
 * random patches and their horizontal reflections; Form 2: PCA-based colour
 * intensity jittering; the paper's section 4.1).  Image n is the P x P patch
 * of source n (side Hs x Ws) whose top-left corner is (y0, x0), mirrored
 * left-right (x -> P-1-x) when flip != 0, and every pixel of channel c gets
 *     sum_i eigvec[c*3 + i] * alpha[n*3 + i] * eigval[i]
 * added: the principal components weighted by the image's draws times their
 * eigenvalues, the same vector for every pixel of the image.  crop[n*3 ..]
 * holds (y0, x0, flip); offsets outside the source are clamped into it (the
 * library's stated rule for out-of-range draws; the pages draw only valid
 * ones).
 * Pinned by: identity case (P = Hs = Ws, zero offsets, no flip, alpha 0),
 * mirror twice, the ten-view crops as special cases, constant images.
 * ------------------------------------------------------------------------ */
void orc_augment(const double* src, int N, int C, int Hs, int Ws, const int32_t* crop, const double* alpha,
                 const double* eigvec, const double* eigval, int P, double* out) {
#pragma omp parallel for
  for (int n = 0; n < N; ++n) {
    int y0 = crop[n * 3], x0 = crop[n * 3 + 1];
    const bool flip = crop[n * 3 + 2] != 0;
    y0 = y0 < 0 ? 0 : (y0 > Hs - P ? Hs - P : y0);
    x0 = x0 < 0 ? 0 : (x0 > Ws - P ? Ws - P : x0);
    for (int c = 0; c < C; ++c) {
      double shift = 0.0;
      for (int i = 0; i < 3; ++i) shift += eigvec[c * 3 + i] * alpha[n * 3 + i] * eigval[i];
      for (int y = 0; y < P; ++y)
        for (int x = 0; x < P; ++x) {
          const int sx = flip ? (P - 1 - x) : x;
          out[(((size_t)n * C + c) * P + y) * P + x] =
              src[(((size_t)n * C + c) * Hs + y0 + y) * Ws + x0 + sx] + shift;
        }
    }
  }
}

/* Mean of the ten views' softmax outputs for each source image. */
void orc_view_mean(const double* p, int N, int O, double* out) {
  for (int n = 0; n < N; ++n)
    for (int i = 0; i < O; ++i) {
      double s = 0.0;
      for (int v = 0; v < 10; ++v) s += p[((size_t)n * 10 + v) * O + i];
      out[(size_t)n * O + i] = s / 10.0;
    }
}

int orc_num_threads(void) {
#ifdef _OPENMP
  return omp_get_max_threads();
#else
  return 1;
#endif
}

}  // extern "C"
