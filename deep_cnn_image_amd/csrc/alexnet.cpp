// C ABI of the AlexNet library: argument validation (host only), the
// workspace plan, and the launch sequences of the forward pass, the ten-view
// forward pass and the training step.
#include <hip/hip_runtime.h>
#include <math.h>
#include <string.h>

#include <atomic>
#include <mutex>

#include "../../include/alexnet.h"
#include "launch.hpp"
#include "plan.hpp"

using namespace ax;

namespace {

inline bool aligned(const void* p, size_t a) { return ((uintptr_t)p & (a - 1)) == 0; }

// Per-device "is gfx950" cache: 0 unknown, 1 yes, 2 no.
std::atomic<int> g_arch_ok[64];

int check_device() {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return ALEXNET_E_HIP;
  if (dev < 0 || dev >= 64) return ALEXNET_E_DEVICE;
  int s = g_arch_ok[dev].load(std::memory_order_relaxed);
  if (s == 0) {
    hipDeviceProp_t prop;
    if (hipGetDeviceProperties(&prop, dev) != hipSuccess) return ALEXNET_E_HIP;
    s = strncmp(prop.gcnArchName, "gfx950", 6) == 0 ? 1 : 2;
    g_arch_ok[dev].store(s, std::memory_order_relaxed);
  }
  return s == 1 ? ALEXNET_OK : ALEXNET_E_DEVICE;
}

// Device scratch of alexnet_forward_noalloc: the whole forward workspace
// (layer-1 staging, re-laid-out weights, activations, split-K partials) of
// any configuration that fits.  One copy per GPU, loaded with the code
// object and held until the process ends; every call on a GPU shares it.
// Host code never passes `scratch` itself to a kernel (on the host it names a
// stand-in, not the device copy): it uses the address hipGetSymbolAddress
// returns for the current device, looked up once per device.
static __device__ __align__(256) unsigned char scratch[ALEXNET_NOALLOC_SCRATCH_BYTES];

std::mutex g_scratch_mu;
void* g_scratch_ptr[64];

int scratch_address(void** out) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return ALEXNET_E_HIP;
  if (dev < 0 || dev >= 64) return ALEXNET_E_DEVICE;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* ptr = nullptr;
    if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)) != hipSuccess || !ptr) return ALEXNET_E_HIP;
    g_scratch_ptr[dev] = ptr;
  }
  *out = g_scratch_ptr[dev];
  return ALEXNET_OK;
}

int check_params(const void* const* params, int n) {
  if (!params) return ALEXNET_E_NULL;
  for (int i = 0; i < n; ++i) {
    if (!params[i]) return ALEXNET_E_NULL;
    if (!aligned(params[i], 16)) return ALEXNET_E_ALIGN;
  }
  return ALEXNET_OK;
}

// Kernel timers of one call, indexed by alexnet_kernel.
struct Timers {
  KTimer t[ALEXNET_KT_COUNT];
  bool on[ALEXNET_KT_COUNT] = {};
  const KTimer* operator()(int id) const { return on[id] ? &t[id] : nullptr; }
};

int load_timers(const alexnet_timer* timers, int32_t n, Timers* out) {
  if (n < 0) return ALEXNET_E_ARG;
  if (n > 0 && !timers) return ALEXNET_E_NULL;
  for (int i = 0; i < n; ++i) {
    const int k = timers[i].kernel;
    if (k < 1 || k >= ALEXNET_KT_COUNT) return ALEXNET_E_ARG;
    if (!timers[i].start || !timers[i].stop) return ALEXNET_E_NULL;
    out->t[k].start = (hipEvent_t)timers[i].start;
    out->t[k].stop = (hipEvent_t)timers[i].stop;
    out->on[k] = true;
  }
  return ALEXNET_OK;
}

inline char* at(void* ws, const Buf& b) { return (char*)ws + b.off; }
inline char* tp(void* ws, const Plan& p, int id) { return (char*)ws + p.tap[id].buf.off; }

#define HIPCHK(x)                                  \
  do {                                             \
    if ((x) != hipSuccess) return ALEXNET_E_HIP;   \
  } while (0)

// What the network head produces after FC8: softmax probabilities (probs may
// be null) and, with labels, the cross-entropy gradient and per-row losses.
struct Head {
  const int32_t* labels;
  float* probs;
  void* dz;
  float* rowloss;
};

// Forward pass.  train: dropout masks of (seed, step); else the 1 - p scale.
// x: 227 x 227 images, 256 x 256 ten-view sources (ten-view plan), or, with
// `aug`, aug_h x aug_w sources of augmented patches.
int enqueue_forward(const Plan& p, const void* const* prm, const void* x, void* ws, bool train,
                    uint64_t seed, uint64_t step, hipStream_t st, const Timers& T, const Head& head,
                    const AugSrc* aug = nullptr, int aug_h = 0, int aug_w = 0) {
  const DType dt = p.cfg.dtype == ALEXNET_BF16 ? BF16 : F32;
  const Net& net = p.net;
  const int N = p.N;
  const alexnet_cfg& c = p.cfg;

  // weights into the layouts the GEMM loaders read (for a training step also
  // the data-gradient layouts of the backward pass), one launch
  {
    WeightPrep jobs[WPREP_MAX];
    int nj = 0;
    jobs[nj++] = WeightPrep{WPREP_W1S, prm[0], at(ws, p.w1s), 96, 3, 11, 1};
    for (int i = 1; i < 5; ++i) {
      const ConvShape& s = net.conv[i];
      jobs[nj++] = WeightPrep{WPREP_KHWC, prm[2 * i], at(ws, p.wr[i]), s.Cout, s.Cin / s.groups, s.K, s.groups};
      if (train)
        jobs[nj++] =
            WeightPrep{WPREP_DGRAD, prm[2 * i], at(ws, p.wt[i]), s.Cout, s.Cin / s.groups, s.K, s.groups};
    }
    // together with the layer-1 input staging
    const bool tenview = p.mode == ALEXNET_MODE_TENVIEW;
    const int kind = aug ? SRC_AUGMENT : tenview ? SRC_TENVIEW : SRC_IMAGES;
    const int hs = aug ? aug_h : tenview ? 256 : 227, wsz = aug ? aug_w : hs;
    HIPCHK(stage_inputs(dt, jobs, nj, x, hs, wsz, kind, aug, N, at(ws, p.xs2d), st, T(ALEXNET_KT_S2D)));
  }
  float* part = (float*)at(ws, p.part);   // split-K partials (small batches, FC layers)
  HIPCHK(conv1_fwd(dt, at(ws, p.xs2d), N, at(ws, p.w1s), prm[1], tp(ws, p, T_CONV1), part, p.part_bytes, st,
                   T(ALEXNET_KT_CONV1_FWD)));
  HIPCHK(lrn_pool_fwd(dt, tp(ws, p, T_CONV1), tp(ws, p, T_POOL1), (uint8_t*)tp(ws, p, T_ARG1),
                      c.lrn_taps ? tp(ws, p, T_LRN1) : nullptr, N, 55, 55, 96, c.lrn_k, c.lrn_alpha, c.lrn_beta,
                      c.lrn_n, st, T(ALEXNET_KT_LRNPOOL1_FWD)));
  HIPCHK(conv_fwd(dt, net.conv[1], tp(ws, p, T_POOL1), at(ws, p.wr[1]), prm[3], tp(ws, p, T_CONV2), part,
                  p.part_bytes, st, T(ALEXNET_KT_CONV2_FWD)));
  HIPCHK(lrn_pool_fwd(dt, tp(ws, p, T_CONV2), tp(ws, p, T_POOL2), (uint8_t*)tp(ws, p, T_ARG2),
                      c.lrn_taps ? tp(ws, p, T_LRN2) : nullptr, N, 27, 27, 256, c.lrn_k, c.lrn_alpha, c.lrn_beta,
                      c.lrn_n, st, T(ALEXNET_KT_LRNPOOL2_FWD)));
  HIPCHK(conv_fwd(dt, net.conv[2], tp(ws, p, T_POOL2), at(ws, p.wr[2]), prm[5], tp(ws, p, T_CONV3), part,
                  p.part_bytes, st, T(ALEXNET_KT_CONV3_FWD)));
  HIPCHK(conv_fwd(dt, net.conv[3], tp(ws, p, T_CONV3), at(ws, p.wr[3]), prm[7], tp(ws, p, T_CONV4), part,
                  p.part_bytes, st, T(ALEXNET_KT_CONV4_FWD)));
  HIPCHK(conv_fwd(dt, net.conv[4], tp(ws, p, T_CONV4), at(ws, p.wr[4]), prm[9], tp(ws, p, T_CONV5), part,
                  p.part_bytes, st, T(ALEXNET_KT_CONV5_FWD)));
  HIPCHK(pool5_fwd(dt, tp(ws, p, T_CONV5), tp(ws, p, T_POOL5), (uint8_t*)tp(ws, p, T_ARG5), N, 13, 13, 256, st,
                   T(ALEXNET_KT_POOL5_FWD)));

  FcEpi ep{};
  ep.relu = 1;
  if (train) {
    ep.drop = 1;
    ep.thresh = (uint32_t)floor((double)c.dropout_p * 4294967296.0);
    ep.seed = seed;
    ep.step = step;
  } else {
    ep.drop = 2;
    ep.scale = 1.f - c.dropout_p;
  }
  ep.layer = 0;
  HIPCHK(fc_fwd(dt, N, 9216, 4096, tp(ws, p, T_POOL5), prm[10], prm[11], ep, tp(ws, p, T_DROP6), nullptr,
                part, p.part_bytes, st, T(ALEXNET_KT_FC6_FWD)));
  ep.layer = 1;
  HIPCHK(fc_fwd(dt, N, 4096, 4096, tp(ws, p, T_DROP6), prm[12], prm[13], ep, tp(ws, p, T_DROP7), nullptr,
                part, p.part_bytes, st, T(ALEXNET_KT_FC7_FWD)));
  HIPCHK(fc_head(dt, N, 4096, 1000, tp(ws, p, T_DROP7), prm[14], prm[15], (float*)tp(ws, p, T_LOGITS),
                 head.labels, head.probs, head.dz, head.rowloss, part, p.part_bytes, st, T(ALEXNET_KT_FC8_FWD)));
  return ALEXNET_OK;
}

// Fork/join of the caller's side stream, with the caller's events.  fork()
// makes the side stream wait for everything enqueued on the main stream so
// far and returns it; join() (also run by the destructor, so an early error
// return still joins) makes the main stream wait for everything enqueued on
// the side stream.  Each fork uses its own event, the join the last one.  If
// a fork cannot be enqueued, the host waits for the side stream and the rest
// of the call runs on the main stream alone.
struct SideFork {
  hipStream_t main = nullptr, side = nullptr;
  void* const* ev = nullptr;
  int n = 0;
  bool used = false;
  SideFork(hipStream_t m, hipStream_t s, void* const* events) : main(m), side(s), ev(events) {}
  hipStream_t fork() {
    if (!side) return main;
    if (n >= ALEXNET_SIDE_EVENTS - 1) return serial();
    hipEvent_t e = (hipEvent_t)ev[n++];
    if (hipEventRecord(e, main) != hipSuccess || hipStreamWaitEvent(side, e, 0) != hipSuccess) return serial();
    used = true;
    return side;
  }
  hipStream_t serial() {
    if (used) hipStreamSynchronize(side);
    side = nullptr;
    used = false;
    return main;
  }
  void join() {
    if (!side || !used) return;
    hipEvent_t e = (hipEvent_t)ev[ALEXNET_SIDE_EVENTS - 1];
    if (hipEventRecord(e, side) != hipSuccess || hipStreamWaitEvent(main, e, 0) != hipSuccess)
      hipStreamSynchronize(side);
    used = false;
  }
  ~SideFork() { join(); }
};

// Backward pass, with the SGD update of every tensor folded in:
//  - FC weights inside their weight-gradient GEMM, after the layer's data
//    gradient has read the old working weights;
//  - conv weights as their split-K gradient is reduced; the layer's data
//    gradient reads the data-gradient copy prepared from the old weights at
//    the start of the step;
//  - biases with their gradients, in the last two launches.
// Every gradient except the FC weights' also lands in the workspace (taps).
// With a side stream, the weight gradients run on it (see below).
int enqueue_backward(const Plan& p, void* const* work, float* const* master, float* const* momentum,
                     const SgdHyper& hy, float* loss, void* ws, hipStream_t st, const Timers& T,
                     hipStream_t side_st, void* const* side_ev) {
  const DType dt = p.cfg.dtype == ALEXNET_BF16 ? BF16 : F32;
  const Net& net = p.net;
  const int N = p.N;
  const alexnet_cfg& c = p.cfg;
  float* part = (float*)at(ws, p.part);
  float* cs = (float*)at(ws, p.colsum);
  auto gw = [&](int i) { return (float*)tp(ws, p, T_GW1 + i); };
  auto gb = [&](int i) { return (float*)tp(ws, p, T_GB1 + i); };

  // FC8: dh7 = dz W8 * [drop7 > 0]   (drop7 > 0 <=> kept and ReLU active)
  HIPCHK(fc_dgrad(dt, N, 4096, 1000, tp(ws, p, T_DLOGITS), work[14], tp(ws, p, T_DROP7), tp(ws, p, T_DFC7),
                  part, p.part_bytes, st, T(ALEXNET_KT_FC8_DGRAD)));
  HIPCHK(fc_wgrad_sgd(dt, N, 4096, 1000, tp(ws, p, T_DLOGITS), tp(ws, p, T_DROP7), hy, master[14],
                      momentum[14], work[14], st, T(ALEXNET_KT_FC8_WGRAD)));
  // FC7
  HIPCHK(fc_dgrad(dt, N, 4096, 4096, tp(ws, p, T_DFC7), work[12], tp(ws, p, T_DROP6), tp(ws, p, T_DFC6),
                  part, p.part_bytes, st, T(ALEXNET_KT_FC7_DGRAD)));
  HIPCHK(fc_wgrad_sgd(dt, N, 4096, 4096, tp(ws, p, T_DFC7), tp(ws, p, T_DROP6), hy, master[12],
                      momentum[12], work[12], st, T(ALEXNET_KT_FC7_WGRAD)));
  // FC6 -> gradient w.r.t. the flattened pool5 output
  HIPCHK(fc_dgrad(dt, N, 9216, 4096, tp(ws, p, T_DFC6), work[10], nullptr, tp(ws, p, T_DFLAT), part,
                  p.part_bytes, st, T(ALEXNET_KT_FC6_DGRAD)));
  HIPCHK(fc_wgrad_sgd(dt, N, 9216, 4096, tp(ws, p, T_DFC6), tp(ws, p, T_POOL5), hy, master[10],
                      momentum[10], work[10], st, T(ALEXNET_KT_FC6_WGRAD)));
  // pool5 backward * ReLU5'
  HIPCHK(pool5_bwd(dt, tp(ws, p, T_DFLAT), (const uint8_t*)tp(ws, p, T_ARG5), tp(ws, p, T_CONV5),
                   tp(ws, p, T_DCONV5), N, 13, 13, 256, st, T(ALEXNET_KT_POOL5_BWD)));
  // conv5, conv4, conv3
  const int din[5] = {-1, T_DIN2, T_DIN3, T_DCONV3, T_DCONV4};
  const int dz[5] = {T_DCONV1, T_DCONV2, T_DCONV3, T_DCONV4, T_DCONV5};
  const int xin[5] = {-1, T_POOL1, T_POOL2, T_CONV3, T_CONV4};
  const int mask[5] = {-1, -1, -1, T_CONV3, T_CONV4};
  const int ktw[5] = {ALEXNET_KT_CONV1_WGRAD, ALEXNET_KT_CONV2_WGRAD, ALEXNET_KT_CONV3_WGRAD,
                      ALEXNET_KT_CONV4_WGRAD, ALEXNET_KT_CONV5_WGRAD};
  const int ktd[5] = {0, ALEXNET_KT_CONV2_DGRAD, ALEXNET_KT_CONV3_DGRAD, ALEXNET_KT_CONV4_DGRAD,
                      ALEXNET_KT_CONV5_DGRAD};
  // Bias gradients with their SGD, in two passes over disjoint parts of the
  // column-sum scratch.  Layers 3-8 read their stored output gradients; all
  // of them are complete once layer 3's is, so that pass follows layer 3's
  // weight gradient (on the side stream, beside the rest of the backward
  // pass, when there is one).  Layers 1 and 2 start from the per-row sums
  // their pool/LRN backward leaves; that pass, with the batch-mean loss, ends
  // the step.
  BiasJob bias_jobs[8];
  {
    const int dys[8] = {T_DCONV1, T_DCONV2, T_DCONV3, T_DCONV4, T_DCONV5, T_DFC6, T_DFC7, T_DLOGITS};
    for (int i = 0; i < 8; ++i) {
      const bool rows_f32 = i < 2;
      const int64_t rows = rows_f32 ? (int64_t)N * net.conv[i].Ho
                           : i < 5  ? (int64_t)N * net.conv[i].Ho * net.conv[i].Wo
                                    : N;
      const void* src = rows_f32 ? (const void*)at(ws, p.bias_rows[i]) : tp(ws, p, dys[i]);
      bias_jobs[i] = BiasJob{src, rows, (int)net.bcount[i], gb(i), master[2 * i + 1], momentum[2 * i + 1],
                             work[2 * i + 1], rows_f32};
    }
  }
  float* const bias_cs12 = cs + bias_grad_scratch_bytes(bias_jobs + 2, 6) / sizeof(float);
  auto bias_pass = [&](const BiasJob* jobs, int first, int n, float* scratch, const float* rowloss,
                       hipStream_t s, const KTimer* kt) {
    return bias_grads_sgd(dt, jobs + first, n, hy, scratch, rowloss, N, loss, s, kt);
  };

  // The conv weight gradients (with their SGD update) need nothing from the
  // data-gradient chain after their own output gradient, and nothing in the
  // chain reads what they write: given a side stream, each is forked onto it
  // once its output gradient is complete, so it runs beside the rest of the
  // backward pass.  Not when a data gradient of the step splits over k (small
  // batches): both would use the split-K region of the workspace.  Timers
  // change nothing in this order: a timed kernel's events go on the stream it
  // runs on, and its time then includes the GPU it shares with the other
  // stream's kernels.
  bool concurrent = side_st != nullptr;
  for (int i = 1; i < 5; ++i)
    if (conv_dgrad_part_bytes(dt, net.conv[i]) != 0) concurrent = false;
  SideFork side(st, concurrent ? side_st : nullptr, side_ev);
  for (int i = 4; i >= 2; --i) {
    const ConvShape& s = net.conv[i];
    const SgdTarget u{master[2 * i], momentum[2 * i], work[2 * i], hy};
    hipStream_t sw = side.fork();
    HIPCHK(conv_wgrad(dt, s, tp(ws, p, dz[i]), tp(ws, p, xin[i]), part, p.part_bytes, gw(i), &u, sw, T(ktw[i])));
    if (i == 2) HIPCHK(bias_pass(bias_jobs, 2, 6, cs, nullptr, sw, T(ALEXNET_KT_BIAS)));
    HIPCHK(conv_dgrad(dt, s, tp(ws, p, dz[i]), at(ws, p.wt[i]), mask[i] >= 0 ? tp(ws, p, mask[i]) : nullptr,
                      tp(ws, p, din[i]), part, p.part_bytes, st, T(ktd[i])));
  }
  // pool2 -> LRN2 -> ReLU2
  HIPCHK(pool_lrn_bwd(dt, tp(ws, p, T_DIN3), (const uint8_t*)tp(ws, p, T_ARG2), tp(ws, p, T_CONV2),
                      tp(ws, p, T_DCONV2), c.lrn_taps ? tp(ws, p, T_DLRN2) : nullptr, (float*)at(ws, p.bias_rows[1]),
                      N, 27, 27, 256, c.lrn_k, c.lrn_alpha, c.lrn_beta, c.lrn_n, st, T(ALEXNET_KT_POOLLRN2_BWD)));
  {
    const ConvShape& s = net.conv[1];
    const SgdTarget u{master[2], momentum[2], work[2], hy};
    hipStream_t sw = side.fork();
    HIPCHK(conv_wgrad(dt, s, tp(ws, p, T_DCONV2), tp(ws, p, T_POOL1), part, p.part_bytes, gw(1), &u, sw,
                      T(ALEXNET_KT_CONV2_WGRAD)));
    HIPCHK(conv_dgrad(dt, s, tp(ws, p, T_DCONV2), at(ws, p.wt[1]), nullptr, tp(ws, p, T_DIN2), part,
                      p.part_bytes, st, T(ALEXNET_KT_CONV2_DGRAD)));
  }
  // pool1 -> LRN1 -> ReLU1, then layer-1 weight gradient (no input gradient)
  HIPCHK(pool_lrn_bwd(dt, tp(ws, p, T_DIN2), (const uint8_t*)tp(ws, p, T_ARG1), tp(ws, p, T_CONV1),
                      tp(ws, p, T_DCONV1), c.lrn_taps ? tp(ws, p, T_DLRN1) : nullptr, (float*)at(ws, p.bias_rows[0]),
                      N, 55, 55, 96, c.lrn_k, c.lrn_alpha, c.lrn_beta, c.lrn_n, st, T(ALEXNET_KT_POOLLRN1_BWD)));
  {
    const SgdTarget u{master[0], momentum[0], work[0], hy};
    hipStream_t sw = side.fork();
    HIPCHK(conv1_wgrad(dt, N, tp(ws, p, T_DCONV1), at(ws, p.xs2d), part, p.part_bytes, gw(0), &u, sw,
                       T(ALEXNET_KT_CONV1_WGRAD)));
  }
  // bias gradients of all eight layers, and their SGD update, in two passes
  HIPCHK(bias_pass(bias_jobs, 0, 2, bias_cs12, (const float*)tp(ws, p, T_ROWLOSS), st, T(ALEXNET_KT_BIAS12)));
  return ALEXNET_OK;
}

int prepare(const alexnet_cfg* cfg, int mode, void* ws, size_t ws_bytes, Plan* p) {
  int r = make_plan(cfg, mode, p);
  if (r != ALEXNET_OK) return r;
  if (!ws) return ALEXNET_E_NULL;
  if (!aligned(ws, 256)) return ALEXNET_E_ALIGN;
  if (ws_bytes < p->total) return ALEXNET_E_WORKSPACE;
  return ALEXNET_OK;
}

}  // namespace

extern "C" {

void alexnet_default_cfg(alexnet_cfg* cfg, int32_t batch, int32_t groups, int32_t dtype) {
  if (!cfg) return;
  cfg->batch = batch;
  cfg->groups = groups;
  cfg->dtype = dtype;
  cfg->lrn_n = 5;
  cfg->lrn_k = 2.f;
  cfg->lrn_alpha = 1e-4f;
  cfg->lrn_beta = 0.75f;
  cfg->dropout_p = 0.5f;
  cfg->lrn_taps = 0;
}

size_t alexnet_workspace_bytes(const alexnet_cfg* cfg, int mode) {
  Plan p;
  return make_plan(cfg, mode, &p) == ALEXNET_OK ? p.total : 0;
}

int alexnet_forward_timed(const alexnet_cfg* cfg, const void* const params[16], const void* x, float* probs,
                          void* ws, size_t ws_bytes, void* stream, const alexnet_timer* timers,
                          int32_t n_timers) {
  Plan p;
  int r = prepare(cfg, ALEXNET_MODE_FORWARD, ws, ws_bytes, &p);
  if (r != ALEXNET_OK) return r;
  if ((r = check_params(params, 16)) != ALEXNET_OK) return r;
  if (!x || !probs) return ALEXNET_E_NULL;
  if (!aligned(x, 16) || !aligned(probs, 16)) return ALEXNET_E_ALIGN;
  Timers T;
  if ((r = load_timers(timers, n_timers, &T)) != ALEXNET_OK) return r;
  if ((r = check_device()) != ALEXNET_OK) return r;
  hipStream_t st = (hipStream_t)stream;
  if ((r = enqueue_forward(p, params, x, ws, false, 0, 0, st, T, Head{nullptr, probs, nullptr, nullptr})) !=
      ALEXNET_OK)
    return r;
  return ALEXNET_OK;
}

int alexnet_forward(const alexnet_cfg* cfg, const void* const params[16], const void* x, float* probs,
                    void* ws, size_t ws_bytes, void* stream) {
  return alexnet_forward_timed(cfg, params, x, probs, ws, ws_bytes, stream, nullptr, 0);
}

int alexnet_forward_noalloc(const alexnet_cfg* cfg, const void* const params[16], const void* x, float* probs,
                            void* stream) {
  Plan p;
  int r = make_plan(cfg, ALEXNET_MODE_FORWARD, &p);
  if (r != ALEXNET_OK) return r;
  if (p.total > ALEXNET_NOALLOC_SCRATCH_BYTES) return ALEXNET_E_SCRATCH;
  if ((r = check_params(params, 16)) != ALEXNET_OK) return r;
  if (!x || !probs) return ALEXNET_E_NULL;
  if (!aligned(x, 16) || !aligned(probs, 16)) return ALEXNET_E_ALIGN;
  if ((r = check_device()) != ALEXNET_OK) return r;
  void* ws = nullptr;
  if ((r = scratch_address(&ws)) != ALEXNET_OK) return r;
  return enqueue_forward(p, params, x, ws, false, 0, 0, (hipStream_t)stream, Timers(),
                         Head{nullptr, probs, nullptr, nullptr});
}

int alexnet_forward_tenview(const alexnet_cfg* cfg, const void* const params[16], const void* src,
                            float* probs, void* ws, size_t ws_bytes, void* stream) {
  Plan p;
  int r = prepare(cfg, ALEXNET_MODE_TENVIEW, ws, ws_bytes, &p);
  if (r != ALEXNET_OK) return r;
  if ((r = check_params(params, 16)) != ALEXNET_OK) return r;
  if (!src || !probs) return ALEXNET_E_NULL;
  if (!aligned(src, 16) || !aligned(probs, 16)) return ALEXNET_E_ALIGN;
  if ((r = check_device()) != ALEXNET_OK) return r;
  hipStream_t st = (hipStream_t)stream;
  float* vp = (float*)tp(ws, p, T_VIEWPROBS);
  if ((r = enqueue_forward(p, params, src, ws, false, 0, 0, st, Timers(), Head{nullptr, vp, nullptr, nullptr})) !=
      ALEXNET_OK)
    return r;
  if (view_mean(vp, probs, cfg->batch, 1000, st) != hipSuccess) return ALEXNET_E_HIP;
  return ALEXNET_OK;
}

}  // extern "C"

namespace {

// Host-side checks of an augmentation description; the crop offsets are
// device data, clamped by the kernels.
int check_augment(const alexnet_augment* aug, int32_t src_h, int32_t src_w, AugSrc* out) {
  if (!aug || !aug->crop || !aug->alpha || !aug->eigval || !aug->eigvec) return ALEXNET_E_NULL;
  if (!aligned(aug->crop, 4) || !aligned(aug->alpha, 4) || !aligned(aug->eigval, 4) || !aligned(aug->eigvec, 4))
    return ALEXNET_E_ALIGN;
  if (src_h < 227 || src_w < 227 || src_h > 8192 || src_w > 8192) return ALEXNET_E_SHAPE;
  *out = AugSrc{aug->crop, aug->alpha, aug->eigvec, aug->eigval};
  return ALEXNET_OK;
}

int train_step_impl(const alexnet_cfg* cfg, float* const master[16], float* const momentum[16],
                    void* const work[16], const void* x, const AugSrc* aug, int aug_h, int aug_w,
                    const int32_t* labels, float lr, float momentum_coef, float weight_decay, uint64_t seed,
                    uint64_t step, float* loss, float* probs, void* ws, size_t ws_bytes, void* stream,
                    const alexnet_exec* ex) {
  const alexnet_timer* timers = ex ? ex->timers : nullptr;
  const int32_t n_timers = ex ? ex->n_timers : 0;
  hipStream_t side_st = ex ? (hipStream_t)ex->side_stream : nullptr;
  if (side_st) {
    if (side_st == (hipStream_t)stream) return ALEXNET_E_ARG;
    for (int i = 0; i < ALEXNET_SIDE_EVENTS; ++i)
      if (!ex->events[i]) return ALEXNET_E_NULL;
  }
  Plan p;
  int r = prepare(cfg, ALEXNET_MODE_TRAIN, ws, ws_bytes, &p);
  if (r != ALEXNET_OK) return r;
  if ((r = check_params((const void* const*)master, 16)) != ALEXNET_OK) return r;
  if ((r = check_params((const void* const*)momentum, 16)) != ALEXNET_OK) return r;
  if ((r = check_params((const void* const*)work, 16)) != ALEXNET_OK) return r;
  if (!x || !labels || !loss) return ALEXNET_E_NULL;
  if (!aligned(x, 16) || !aligned(labels, 4) || !aligned(loss, 4)) return ALEXNET_E_ALIGN;
  if (probs && !aligned(probs, 16)) return ALEXNET_E_ALIGN;
  if (!isfinite(lr) || !isfinite(momentum_coef) || !isfinite(weight_decay)) return ALEXNET_E_ARG;
  Timers T;
  if ((r = load_timers(timers, n_timers, &T)) != ALEXNET_OK) return r;
  if ((r = check_device()) != ALEXNET_OK) return r;
  hipStream_t st = (hipStream_t)stream;
  const Head head{labels, probs, tp(ws, p, T_DLOGITS), (float*)tp(ws, p, T_ROWLOSS)};
  if ((r = enqueue_forward(p, (const void* const*)work, x, ws, true, seed, step, st, T, head, aug, aug_h,
                           aug_w)) != ALEXNET_OK)
    return r;
  const SgdHyper hy{lr, momentum_coef, weight_decay * lr};
  if ((r = enqueue_backward(p, work, master, momentum, hy, loss, ws, st, T, side_st,
                            side_st ? ex->events : nullptr)) != ALEXNET_OK)
    return r;
  return ALEXNET_OK;
}

}  // namespace

extern "C" {

int alexnet_train_step_ex(const alexnet_cfg* cfg, float* const master[16], float* const momentum[16],
                          void* const work[16], const void* x, const alexnet_augment* aug, int32_t src_h,
                          int32_t src_w, const int32_t* labels, float lr, float momentum_coef,
                          float weight_decay, uint64_t seed, uint64_t step, float* loss, float* probs, void* ws,
                          size_t ws_bytes, void* stream, const alexnet_exec* ex) {
  if (!aug)
    return train_step_impl(cfg, master, momentum, work, x, nullptr, 0, 0, labels, lr, momentum_coef,
                           weight_decay, seed, step, loss, probs, ws, ws_bytes, stream, ex);
  AugSrc a;
  const int r = check_augment(aug, src_h, src_w, &a);
  if (r != ALEXNET_OK) return r;
  return train_step_impl(cfg, master, momentum, work, x, &a, src_h, src_w, labels, lr, momentum_coef,
                         weight_decay, seed, step, loss, probs, ws, ws_bytes, stream, ex);
}

int alexnet_train_step_timed(const alexnet_cfg* cfg, float* const master[16], float* const momentum[16],
                             void* const work[16], const void* x, const int32_t* labels, float lr,
                             float momentum_coef, float weight_decay, uint64_t seed, uint64_t step,
                             float* loss, float* probs, void* ws, size_t ws_bytes, void* stream,
                             const alexnet_timer* timers, int32_t n_timers) {
  alexnet_exec ex{};
  ex.timers = timers;
  ex.n_timers = n_timers;
  return alexnet_train_step_ex(cfg, master, momentum, work, x, nullptr, 0, 0, labels, lr, momentum_coef,
                               weight_decay, seed, step, loss, probs, ws, ws_bytes, stream, &ex);
}

int alexnet_train_step_augmented_timed(const alexnet_cfg* cfg, float* const master[16],
                                       float* const momentum[16], void* const work[16], const void* src,
                                       int32_t src_h, int32_t src_w, const alexnet_augment* aug,
                                       const int32_t* labels, float lr, float momentum_coef, float weight_decay,
                                       uint64_t seed, uint64_t step, float* loss, float* probs, void* ws,
                                       size_t ws_bytes, void* stream, const alexnet_timer* timers,
                                       int32_t n_timers) {
  if (!aug) return ALEXNET_E_NULL;
  alexnet_exec ex{};
  ex.timers = timers;
  ex.n_timers = n_timers;
  return alexnet_train_step_ex(cfg, master, momentum, work, src, aug, src_h, src_w, labels, lr, momentum_coef,
                               weight_decay, seed, step, loss, probs, ws, ws_bytes, stream, &ex);
}

int alexnet_train_step_augmented(const alexnet_cfg* cfg, float* const master[16], float* const momentum[16],
                                 void* const work[16], const void* src, int32_t src_h, int32_t src_w,
                                 const alexnet_augment* aug, const int32_t* labels, float lr, float momentum_coef,
                                 float weight_decay, uint64_t seed, uint64_t step, float* loss, float* probs,
                                 void* ws, size_t ws_bytes, void* stream) {
  return alexnet_train_step_augmented_timed(cfg, master, momentum, work, src, src_h, src_w, aug, labels, lr,
                                            momentum_coef, weight_decay, seed, step, loss, probs, ws, ws_bytes,
                                            stream, nullptr, 0);
}

int alexnet_augment_images(const alexnet_cfg* cfg, const void* src, int32_t src_h, int32_t src_w,
                           const alexnet_augment* aug, void* x, void* stream) {
  Plan p;
  int r = make_plan(cfg, ALEXNET_MODE_TRAIN, &p);
  if (r != ALEXNET_OK) return r;
  AugSrc a;
  if ((r = check_augment(aug, src_h, src_w, &a)) != ALEXNET_OK) return r;
  if (!src || !x) return ALEXNET_E_NULL;
  if (!aligned(src, 16) || !aligned(x, 16)) return ALEXNET_E_ALIGN;
  if ((r = check_device()) != ALEXNET_OK) return r;
  const DType dt = cfg->dtype == ALEXNET_BF16 ? BF16 : F32;
  return augment_images(dt, src, src_h, src_w, a, cfg->batch, x, (hipStream_t)stream) == hipSuccess
             ? ALEXNET_OK
             : ALEXNET_E_HIP;
}

size_t alexnet_rgb_pca_workspace_bytes(void) { return rgb_pca_scratch_bytes(); }

int alexnet_rgb_pca_timed(const alexnet_cfg* cfg, const void* images, int32_t n, int32_t h, int32_t w,
                          float* eigval, float* eigvec, void* ws, size_t ws_bytes, void* stream,
                          const alexnet_timer* timers, int32_t n_timers) {
  if (!cfg || !images || !eigval || !eigvec || !ws) return ALEXNET_E_NULL;
  if (cfg->dtype != ALEXNET_F32 && cfg->dtype != ALEXNET_BF16) return ALEXNET_E_DTYPE;
  if (n < 1 || h < 1 || w < 1 || (int64_t)n * h * w > ((int64_t)1 << 40)) return ALEXNET_E_SHAPE;
  if (!aligned(images, 16) || !aligned(eigval, 4) || !aligned(eigvec, 4) || !aligned(ws, 256))
    return ALEXNET_E_ALIGN;
  if (ws_bytes < rgb_pca_scratch_bytes()) return ALEXNET_E_WORKSPACE;
  Timers T;
  int r = load_timers(timers, n_timers, &T);
  if (r != ALEXNET_OK) return r;
  if ((r = check_device()) != ALEXNET_OK) return r;
  const DType dt = cfg->dtype == ALEXNET_BF16 ? BF16 : F32;
  return rgb_pca(dt, images, n, h, w, eigval, eigvec, ws, (hipStream_t)stream, T(ALEXNET_KT_RGB_PCA)) ==
                 hipSuccess
             ? ALEXNET_OK
             : ALEXNET_E_HIP;
}

int alexnet_rgb_pca(const alexnet_cfg* cfg, const void* images, int32_t n, int32_t h, int32_t w, float* eigval,
                    float* eigvec, void* ws, size_t ws_bytes, void* stream) {
  return alexnet_rgb_pca_timed(cfg, images, n, h, w, eigval, eigvec, ws, ws_bytes, stream, nullptr, 0);
}

int alexnet_train_step(const alexnet_cfg* cfg, float* const master[16], float* const momentum[16],
                       void* const work[16], const void* x, const int32_t* labels, float lr,
                       float momentum_coef, float weight_decay, uint64_t seed, uint64_t step, float* loss,
                       float* probs, void* ws, size_t ws_bytes, void* stream) {
  return alexnet_train_step_timed(cfg, master, momentum, work, x, labels, lr, momentum_coef, weight_decay,
                                  seed, step, loss, probs, ws, ws_bytes, stream, nullptr, 0);
}

int alexnet_cast_weights(const alexnet_cfg* cfg, float* const master[16], void* const work[16], void* stream) {
  Plan p;
  int r = make_plan(cfg, ALEXNET_MODE_FORWARD, &p);
  if (r != ALEXNET_OK) return r;
  if ((r = check_params((const void* const*)master, 16)) != ALEXNET_OK) return r;
  if ((r = check_params((const void* const*)work, 16)) != ALEXNET_OK) return r;
  if ((r = check_device()) != ALEXNET_OK) return r;
  TensorSet ts;
  for (int i = 0; i < 8; ++i) {
    ts.master[2 * i] = master[2 * i];
    ts.master[2 * i + 1] = master[2 * i + 1];
    ts.work[2 * i] = work[2 * i];
    ts.work[2 * i + 1] = work[2 * i + 1];
    ts.n[2 * i] = p.net.wcount[i];
    ts.n[2 * i + 1] = p.net.bcount[i];
  }
  const DType dt = cfg->dtype == ALEXNET_BF16 ? BF16 : F32;
  return cast_weights(dt, ts, (hipStream_t)stream) == hipSuccess ? ALEXNET_OK : ALEXNET_E_HIP;
}

int alexnet_dropout_mask(uint64_t seed, uint64_t step, int32_t layer, int32_t rows, int32_t cols, float p,
                         uint8_t* mask, void* stream) {
  if (!mask) return ALEXNET_E_NULL;
  if (rows < 0 || cols < 0 || cols % 4 != 0 || layer < 0) return ALEXNET_E_SHAPE;
  if (!aligned(mask, 4)) return ALEXNET_E_ALIGN;
  if (!(p >= 0.f && p < 1.f)) return ALEXNET_E_ARG;
  if ((int64_t)rows * cols == 0) return ALEXNET_OK;
  int r = check_device();
  if (r != ALEXNET_OK) return r;
  const uint32_t thresh = (uint32_t)floor((double)p * 4294967296.0);
  return ax::dropout_mask(seed, step, layer, rows, cols, thresh, mask, (hipStream_t)stream) == hipSuccess
             ? ALEXNET_OK
             : ALEXNET_E_HIP;
}

int alexnet_tap(const alexnet_cfg* cfg, int mode, int tap_id, size_t* offset, int64_t shape[4], int* dtype,
                int* layout) {
  if (!offset || !shape || !dtype || !layout) return ALEXNET_E_NULL;
  Plan p;
  int r = make_plan(cfg, mode, &p);
  if (r != ALEXNET_OK) return r;
  if (tap_id < 0 || tap_id >= T_COUNT || !p.tap[tap_id].present) return ALEXNET_E_ARG;
  const TapDesc& t = p.tap[tap_id];
  *offset = t.buf.off;
  for (int i = 0; i < 4; ++i) shape[i] = t.shape[i];
  *dtype = t.dtype;
  *layout = t.layout;
  return ALEXNET_OK;
}

int alexnet_event_create(int32_t timing, void** event) {
  if (!event) return ALEXNET_E_NULL;
  *event = nullptr;
  hipEvent_t e;
  const unsigned flags = hipEventDisableSystemFence | (timing ? 0u : (unsigned)hipEventDisableTiming);
  if (hipEventCreateWithFlags(&e, flags) != hipSuccess) return ALEXNET_E_HIP;
  *event = e;
  return ALEXNET_OK;
}

int alexnet_event_destroy(void* event) {
  if (!event) return ALEXNET_E_NULL;
  return hipEventDestroy((hipEvent_t)event) == hipSuccess ? ALEXNET_OK : ALEXNET_E_HIP;
}

int alexnet_event_elapsed_ms(void* start, void* stop, float* ms) {
  if (!start || !stop || !ms) return ALEXNET_E_NULL;
  return hipEventElapsedTime(ms, (hipEvent_t)start, (hipEvent_t)stop) == hipSuccess ? ALEXNET_OK : ALEXNET_E_HIP;
}

int alexnet_tap_count(void) { return T_COUNT; }
const char* alexnet_tap_name(int tap_id) { return tap_name(tap_id); }

const char* alexnet_status_string(int s) {
  switch (s) {
    case ALEXNET_OK: return "ok";
    case ALEXNET_E_NULL: return "null pointer";
    case ALEXNET_E_SHAPE: return "batch or groups out of range";
    case ALEXNET_E_DTYPE: return "unsupported dtype";
    case ALEXNET_E_WORKSPACE: return "workspace too small";
    case ALEXNET_E_ALIGN: return "misaligned pointer";
    case ALEXNET_E_DEVICE: return "device is not gfx950";
    case ALEXNET_E_HIP: return "HIP error while enqueueing";
    case ALEXNET_E_ARG: return "invalid argument";
    case ALEXNET_E_SCRATCH: return "configuration needs more than the no-allocation entry point's static scratch";
    default: return "unknown status";
  }
}

}  // extern "C"
