// Workspace plan of one AlexNet call: where every activation, gradient and
// scratch buffer lives in the caller's workspace.  Host only; no HIP calls.
#pragma once
#include <stddef.h>
#include <stdint.h>

#include "../../include/alexnet.h"
#include "launch.hpp"

namespace ax {

struct Buf {
  size_t off = 0, bytes = 0;
};

enum Tap {
  T_CONV1, T_LRN1, T_POOL1, T_ARG1, T_CONV2, T_LRN2, T_POOL2, T_ARG2, T_CONV3, T_CONV4, T_CONV5,
  T_POOL5, T_ARG5, T_DROP6, T_DROP7, T_LOGITS, T_VIEWPROBS,
  T_DLOGITS, T_DFC7, T_DFC6, T_DFLAT, T_DCONV5, T_DCONV4, T_DCONV3, T_DIN3, T_DLRN2, T_DCONV2,
  T_DIN2, T_DLRN1, T_DCONV1,
  T_GW1, T_GW2, T_GW3, T_GW4, T_GW5, T_GW6, T_GW7, T_GW8,
  T_GB1, T_GB2, T_GB3, T_GB4, T_GB5, T_GB6, T_GB7, T_GB8,
  T_ROWLOSS,
  T_COUNT
};

struct TapDesc {
  Buf buf;
  int64_t shape[4];
  int dtype;   // alexnet_dtype
  int layout;  // 0 NHWC, 1 row-major, 2 weight gradient
  bool present;
};

// Geometry of the five convolutions for a forward batch N and group count G.
struct Net {
  int N, G;
  ConvShape conv[5];
  int64_t wcount[8], bcount[8];   // parameter element counts
};
void net_shapes(int N, int G, Net* net);

struct Plan {
  alexnet_cfg cfg;
  int mode;
  int N;          // images through the network (ten-view: 10 * batch)
  int esz;        // bytes per activation element
  Net net;
  Buf xs2d, w1s, wr[5], wt[5];   // layer-1 blocks, re-laid-out weights
  TapDesc tap[T_COUNT];
  Buf part, colsum;
  Buf bias_rows[2];   // training: layers 1 and 2's bias gradients per row of dconv (fp32 [N * H][C])
  size_t part_bytes = 0, colsum_bytes = 0;
  size_t total = 0;
};

// Returns ALEXNET_OK and fills *p, or an error status if cfg/mode are invalid.
int make_plan(const alexnet_cfg* cfg, int mode, Plan* p);
const char* tap_name(int id);

}  // namespace ax
