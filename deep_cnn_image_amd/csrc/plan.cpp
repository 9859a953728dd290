// Workspace plan: shapes of the network, offsets of every buffer, tap table.
#include "plan.hpp"

#include <string.h>

namespace ax {

static const char* const kTapNames[T_COUNT] = {
    "conv1", "lrn1", "pool1", "arg1", "conv2", "lrn2", "pool2", "arg2", "conv3", "conv4", "conv5",
    "pool5", "arg5", "drop6", "drop7", "logits", "view_probs",
    "dlogits", "dfc7", "dfc6", "dflat", "dconv5", "dconv4", "dconv3", "din3", "dlrn2", "dconv2",
    "din2", "dlrn1", "dconv1",
    "gw1", "gw2", "gw3", "gw4", "gw5", "gw6", "gw7", "gw8",
    "gb1", "gb2", "gb3", "gb4", "gb5", "gb6", "gb7", "gb8",
    "rowloss"};

const char* tap_name(int id) { return (id >= 0 && id < T_COUNT) ? kTapNames[id] : nullptr; }

void net_shapes(int N, int G, Net* net) {
  net->N = N;
  net->G = G;
  // (H, Cin, Cout, K, stride, pad, grouped) -- layer list of the pages
  const int H[5] = {227, 27, 13, 13, 13};
  const int Cin[5] = {3, 96, 256, 384, 384};
  const int Cout[5] = {96, 256, 384, 384, 256};
  const int K[5] = {11, 5, 3, 3, 3};
  const int S[5] = {4, 1, 1, 1, 1};
  const int P[5] = {0, 2, 1, 1, 1};
  const bool grouped[5] = {false, true, false, true, true};
  for (int i = 0; i < 5; ++i) {
    ConvShape& c = net->conv[i];
    c.Nimg = N; c.H = H[i]; c.W = H[i]; c.Cin = Cin[i]; c.Cout = Cout[i]; c.K = K[i];
    c.stride = S[i]; c.pad = P[i]; c.groups = grouped[i] ? G : 1;
    c.Ho = (c.H + 2 * c.pad - c.K) / c.stride + 1;
    c.Wo = c.Ho;
    net->wcount[i] = (int64_t)c.Cout * (c.Cin / c.groups) * c.K * c.K;
    net->bcount[i] = c.Cout;
  }
  const int fin[3] = {9216, 4096, 4096}, fout[3] = {4096, 4096, 1000};
  for (int i = 0; i < 3; ++i) {
    net->wcount[5 + i] = (int64_t)fin[i] * fout[i];
    net->bcount[5 + i] = fout[i];
  }
}

namespace {
struct Alloc {
  size_t cur = 0;
  Buf take(size_t bytes) {
    Buf b;
    b.off = cur;
    b.bytes = bytes;
    cur += (bytes + 255) & ~(size_t)255;
    return b;
  }
};
size_t mx(size_t a, size_t b) { return a > b ? a : b; }
}  // namespace

int make_plan(const alexnet_cfg* cfg, int mode, Plan* p) {
  if (!cfg || !p) return ALEXNET_E_NULL;
  if (mode < ALEXNET_MODE_FORWARD || mode > ALEXNET_MODE_TENVIEW) return ALEXNET_E_ARG;
  if (cfg->dtype != ALEXNET_F32 && cfg->dtype != ALEXNET_BF16) return ALEXNET_E_DTYPE;
  if (cfg->groups != 1 && cfg->groups != 2) return ALEXNET_E_SHAPE;
  const int maxb = mode == ALEXNET_MODE_TENVIEW ? 512 : 4096;
  if (cfg->batch < 1 || cfg->batch > maxb) return ALEXNET_E_SHAPE;
  // LRN window: odd, half-width <= 4 (the backward kernel's reach)
  if (cfg->lrn_n < 1 || cfg->lrn_n > 9 || (cfg->lrn_n & 1) == 0) return ALEXNET_E_ARG;
  if (cfg->lrn_taps != 0 && cfg->lrn_taps != 1) return ALEXNET_E_ARG;
  if (!(cfg->lrn_k > 0.f) || !(cfg->lrn_alpha >= 0.f) || !(cfg->lrn_beta >= 0.f)) return ALEXNET_E_ARG;
  if (!(cfg->dropout_p >= 0.f && cfg->dropout_p < 1.f)) return ALEXNET_E_ARG;

  memset(p, 0, sizeof(*p));
  p->cfg = *cfg;
  p->mode = mode;
  const int N = mode == ALEXNET_MODE_TENVIEW ? cfg->batch * 10 : cfg->batch;
  p->N = N;
  p->esz = cfg->dtype == ALEXNET_BF16 ? 2 : 4;
  const int dt = cfg->dtype;
  net_shapes(N, cfg->groups, &p->net);
  const Net& net = p->net;
  const size_t e = p->esz;
  const bool train = mode == ALEXNET_MODE_TRAIN;

  Alloc a;
  // layer-1 input as 4x4 pixel blocks, and re-laid-out working weights
  p->xs2d = a.take((size_t)N * S2D_ELEMS * e);
  p->w1s = a.take(S2D_W_ELEMS * e);
  for (int i = 1; i < 5; ++i) {
    p->wr[i] = a.take((size_t)net.wcount[i] * e);
    if (train) p->wt[i] = a.take((size_t)net.wcount[i] * e);
  }

  auto nhwc = [&](int id, int H, int C, int dtype) {
    TapDesc& t = p->tap[id];
    const size_t es = dtype == ALEXNET_U8 ? 1 : (dtype == ALEXNET_F32 ? 4 : 2);
    t.buf = a.take((size_t)N * H * H * C * es);
    t.shape[0] = N; t.shape[1] = H; t.shape[2] = H; t.shape[3] = C;
    t.dtype = dtype; t.layout = 0; t.present = true;
  };
  auto mat = [&](int id, int64_t rows, int64_t cols, int dtype) {
    TapDesc& t = p->tap[id];
    const size_t es = dtype == ALEXNET_U8 ? 1 : (dtype == ALEXNET_F32 ? 4 : 2);
    t.buf = a.take((size_t)rows * cols * es);
    t.shape[0] = rows; t.shape[1] = cols; t.shape[2] = 1; t.shape[3] = 1;
    t.dtype = dtype; t.layout = 1; t.present = true;
  };

  nhwc(T_CONV1, 55, 96, dt);
  if (cfg->lrn_taps) nhwc(T_LRN1, 55, 96, dt);
  nhwc(T_POOL1, 27, 96, dt);
  nhwc(T_ARG1, 27, 96, ALEXNET_U8);
  nhwc(T_CONV2, 27, 256, dt);
  if (cfg->lrn_taps) nhwc(T_LRN2, 27, 256, dt);
  nhwc(T_POOL2, 13, 256, dt);
  nhwc(T_ARG2, 13, 256, ALEXNET_U8);
  nhwc(T_CONV3, 13, 384, dt);
  nhwc(T_CONV4, 13, 384, dt);
  nhwc(T_CONV5, 13, 256, dt);
  mat(T_POOL5, N, 9216, dt);
  nhwc(T_ARG5, 6, 256, ALEXNET_U8);
  mat(T_DROP6, N, 4096, dt);
  mat(T_DROP7, N, 4096, dt);
  mat(T_LOGITS, N, 1000, ALEXNET_F32);
  if (mode == ALEXNET_MODE_TENVIEW) mat(T_VIEWPROBS, N, 1000, ALEXNET_F32);

  size_t part = mx(mx(fc_fwd_part_bytes(N, 9216, 4096), fc_fwd_part_bytes(N, 4096, 4096)),
                   fc_fwd_part_bytes(N, 4096, 1000));
  const DType ddt = dt == ALEXNET_BF16 ? BF16 : F32;
  part = mx(part, conv1_fwd_part_bytes(ddt, N));
  for (int i = 1; i < 5; ++i) part = mx(part, conv_fwd_part_bytes(ddt, net.conv[i]));
  size_t cs = 0;
  if (train) {
    mat(T_DLOGITS, N, 1000, dt);
    mat(T_DFC7, N, 4096, dt);
    mat(T_DFC6, N, 4096, dt);
    mat(T_DFLAT, N, 9216, dt);
    nhwc(T_DCONV5, 13, 256, dt);
    nhwc(T_DCONV4, 13, 384, dt);
    nhwc(T_DCONV3, 13, 384, dt);
    nhwc(T_DIN3, 13, 256, dt);
    if (cfg->lrn_taps) nhwc(T_DLRN2, 27, 256, dt);
    nhwc(T_DCONV2, 27, 256, dt);
    nhwc(T_DIN2, 27, 96, dt);
    if (cfg->lrn_taps) nhwc(T_DLRN1, 55, 96, dt);
    nhwc(T_DCONV1, 55, 96, dt);
    for (int i = 0; i < 8; ++i) {
      // FC weight gradients are applied inside their GEMM (never stored):
      // no gw6..gw8 taps.
      if (i < 5) {
        TapDesc& w = p->tap[T_GW1 + i];
        w.buf = a.take((size_t)net.wcount[i] * 4);
        const ConvShape& c = net.conv[i];
        w.shape[0] = c.Cout; w.shape[1] = c.Cin / c.groups; w.shape[2] = c.K; w.shape[3] = c.K;
        w.dtype = ALEXNET_F32; w.layout = 2; w.present = true;
      }
      TapDesc& b = p->tap[T_GB1 + i];
      b.buf = a.take((size_t)net.bcount[i] * 4);
      b.shape[0] = net.bcount[i]; b.shape[1] = 1; b.shape[2] = 1; b.shape[3] = 1;
      b.dtype = ALEXNET_F32; b.layout = 1; b.present = true;
    }
    mat(T_ROWLOSS, N, 1, ALEXNET_F32);
    part = mx(part, fc_dgrad_part_bytes(N, 4096, 1000));
    part = mx(part, fc_dgrad_part_bytes(N, 4096, 4096));
    part = mx(part, fc_dgrad_part_bytes(N, 9216, 4096));
    part = mx(part, conv1_wgrad_part_bytes(ddt, N));
    for (int i = 1; i < 5; ++i) {
      part = mx(part, conv_wgrad_part_bytes(net.conv[i]));
      part = mx(part, conv_dgrad_part_bytes(ddt, net.conv[i]));
    }
    // bias-gradient partials of all eight layers at once; layers 1 and 2
    // start from the per-row sums their pool/LRN backward leaves
    for (int i = 0; i < 2; ++i) p->bias_rows[i] = a.take((size_t)N * net.conv[i].Ho * net.conv[i].Cout * 4);
    BiasJob bj[8] = {};
    for (int i = 0; i < 8; ++i) {
      bj[i].rows = i < 2 ? (int64_t)N * net.conv[i].Ho : i < 5 ? (int64_t)N * net.conv[i].Ho * net.conv[i].Wo : N;
      bj[i].C = (int)net.bcount[i];
      bj[i].f32 = i < 2;
    }
    cs = bias_grad_scratch_bytes(bj, 8);
  }
  p->part = a.take(part);
  p->part_bytes = part;
  p->colsum = a.take(cs);
  p->colsum_bytes = cs;
  p->total = a.cur;
  return ALEXNET_OK;
}

}  // namespace ax
