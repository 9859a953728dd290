/*
 * alexnet.h -- C ABI of the MI355X (gfx950) AlexNet forward / training-step
 * library (libalexnet.so).
 *
 * The network is the eight-learned-layer net of Krizhevsky, Sutskever and
 * Hinton (NeurIPS 2012) as described on the paper-graph-ui summary ("Overall
 * Architecture (Layer-by-Layer Specification)", "ReLU Nonlinearity", "Local
 * Response Normalization", "Overlapping Pooling", "Dropout", "Training
 * Procedure Details") and the fermi.ai wiki (layer list with paddings,
 * ALEXNET_FORWARD / TRAIN_STEP):
 *
 *   conv1 96@11x11/s4/p0 -> ReLU -> LRN -> maxpool 3/s2
 *   conv2 256@5x5/p2     -> ReLU -> LRN -> maxpool 3/s2     (groups 1 or 2)
 *   conv3 384@3x3/p1 -> ReLU;  conv4 384@3x3/p1 -> ReLU      (conv4 groups 1 or 2)
 *   conv5 256@3x3/p1 -> ReLU -> maxpool 3/s2 -> flatten (c,h,w) = 9216 (groups 1 or 2)
 *   fc6 9216->4096 -> ReLU -> dropout;  fc7 4096->4096 -> ReLU -> dropout
 *   fc8 4096->1000 -> softmax
 *
 * The paper's two-GPU split with same-GPU connectivity in layers 2, 4 and 5
 * is expressed on one GPU as groups = 2 on conv2, conv4 and conv5.
 *
 * Conventions for every entry point
 *  - Tensors are dense, row-major.  Images are NCHW [N][3][227][227] (ten-view
 *    sources [N][3][256][256]); conv weights OIHW [Cout][Cin/G][k][k]; FC
 *    weights [out][in]; biases [out].
 *  - "params" is an array of 16 device pointers in the order
 *    w1, b1, w2, b2, ..., w8, b8.
 *  - Element type of images, params and work weights is cfg->dtype (fp32 or
 *    bf16 bit patterns); master weights, momentum, probabilities and the loss
 *    are fp32; labels are int32 in [0, 1000).
 *  - All pointers are device pointers unless stated otherwise and must be
 *    16-byte aligned; the workspace must be 256-byte aligned.  The caller owns
 *    every buffer, including the workspace, and every stream and event.  The
 *    library allocates no memory and creates no streams or events of its
 *    own (alexnet_event_create makes an event for the caller, who owns it);
 *    the only state it keeps between calls is a per-device cache of whether the
 *    device is a gfx950 (a fixed fact once read).  Calls are reentrant given
 *    distinct workspaces (and, for alexnet_train_step_ex, distinct side
 *    streams and events).  alexnet_forward_noalloc is the exception: its
 *    workspace is a static device array, one per GPU, and it caches that
 *    array's address per device.
 *  - Calls validate their arguments on the host before any launch and return
 *    an alexnet_status; on error nothing is enqueued.  Work is enqueued on
 *    `stream` (a hipStream_t, 0 = the default stream) and runs
 *    asynchronously; device faults surface at the caller's synchronisation.
 *    Only alexnet_train_step_ex uses a second stream, the caller's, and joins
 *    it back to `stream` before returning, so all of a call's work is ordered
 *    before anything the caller enqueues on `stream` afterwards.
 *  - Activations, gradients and working weights are stored in cfg->dtype;
 *    every sum accumulates in fp32.
 */
#ifndef ALEXNET_H
#define ALEXNET_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  ALEXNET_OK = 0,
  ALEXNET_E_NULL = -1,      /* a required pointer is null                      */
  ALEXNET_E_SHAPE = -2,     /* batch or groups out of range                    */
  ALEXNET_E_DTYPE = -3,     /* dtype not F32/BF16                              */
  ALEXNET_E_WORKSPACE = -4, /* workspace smaller than alexnet_workspace_bytes  */
  ALEXNET_E_ALIGN = -5,     /* pointer misaligned                              */
  ALEXNET_E_DEVICE = -6,    /* current device is not gfx950                    */
  ALEXNET_E_HIP = -7,       /* a HIP call failed while enqueueing              */
  ALEXNET_E_ARG = -8,       /* other invalid argument (mode, tap id, LRN size) */
  ALEXNET_E_SCRATCH = -9    /* alexnet_forward_noalloc: the configuration's
                               workspace exceeds ALEXNET_NOALLOC_SCRATCH_BYTES */
} alexnet_status;

typedef enum { ALEXNET_F32 = 0, ALEXNET_BF16 = 1, ALEXNET_U8 = 2 } alexnet_dtype;

typedef enum {
  ALEXNET_MODE_FORWARD = 0, /* inference forward pass (dropout off, x0.5 scale) */
  ALEXNET_MODE_TRAIN = 1,   /* training step                                   */
  ALEXNET_MODE_TENVIEW = 2  /* ten-view inference over 256x256 sources          */
} alexnet_mode;

typedef struct {
  int32_t batch;     /* images per call; ten-view: source images (10 views each). 1..4096 */
  int32_t groups;    /* 1 = single tower; 2 = conv2/conv4/conv5 split in two groups    */
  int32_t dtype;     /* ALEXNET_F32 or ALEXNET_BF16                                    */
  int32_t lrn_n;     /* LRN window (odd, 1..9), 5 on the pages                         */
  float lrn_k;       /* 2                                                              */
  float lrn_alpha;   /* 1e-4, multiplies the window sum of squares directly            */
  float lrn_beta;    /* 0.75                                                           */
  float dropout_p;   /* 0.5: training drop probability; inference scales by 1 - p      */
  int32_t lrn_taps;  /* 0: LRN and the max-pool after it run fused (forward and
                        backward) and the LRN outputs and their gradients are never
                        stored; 1: they are also stored as taps lrn1, lrn2, dlrn1,
                        dlrn2 (for layer-by-layer checks; results are identical)    */
} alexnet_cfg;

/* Fills *cfg with the pages' constants: k = 2, n = 5, alpha = 1e-4,
 * beta = 0.75, dropout p = 0.5; lrn_taps = 0. */
void alexnet_default_cfg(alexnet_cfg* cfg, int32_t batch, int32_t groups, int32_t dtype);

/* Workspace bytes for one call in `mode`; 0 if cfg is invalid.  Host only. */
size_t alexnet_workspace_bytes(const alexnet_cfg* cfg, int mode);

/* Inference forward pass (fermi.ai ALEXNET_FORWARD; paper-graph-ui layer list,
 * test-time dropout rule of paper-graph-ui "Dropout": inference keeps every
 * unit and scales the FC6/FC7 outputs by 0.5).
 *   x     [batch][3][227][227] cfg->dtype
 *   probs [batch][1000] fp32 softmax output (written) */
int alexnet_forward(const alexnet_cfg* cfg, const void* const params[16], const void* x,
                    float* probs, void* ws, size_t ws_bytes, void* stream);

/* alexnet_forward for callers that cannot allocate device memory (code under
 * HIP graph capture, tight serving loops, harnesses that forbid hipMalloc):
 * the same computation and results, bit for bit, with no workspace argument.
 * The workspace lives in a static device array of ALEXNET_NOALLOC_SCRATCH_BYTES
 * (64 MiB) that each GPU the library runs on holds until the process ends.
 * A configuration whose forward workspace (alexnet_workspace_bytes with
 * ALEXNET_MODE_FORWARD) exceeds it is rejected with ALEXNET_E_SCRATCH before
 * anything is enqueued: fp32 and bf16 up to batch 8 fit.  The call allocates
 * nothing; on the first call on a device it looks up that device's copy of the
 * array (hipGetSymbolAddress).  Every call on one GPU shares the array, so
 * calls that overlap on one GPU (on different streams, or from several host
 * threads without ordering) race; calls ordered on one stream do not.  The
 * array keeps the last call's contents; each call writes every part it reads. */
#define ALEXNET_NOALLOC_SCRATCH_BYTES ((size_t)64 << 20)
int alexnet_forward_noalloc(const alexnet_cfg* cfg, const void* const params[16], const void* x,
                            float* probs, void* stream);

/* Ten-patch test-time averaging (paper-graph-ui "Data Augmentation": the four
 * corner 227x227 patches and the centre patch, each also mirrored, softmax
 * outputs averaged).  View v of source n is batch row n*10 + v; views 0..4 are
 * offsets (0,0), (0,29), (29,0), (29,29), (14,14) as (y,x), views 5..9 the
 * same patches mirrored left-right.  The crops are read directly by layer 1.
 *   src   [batch][3][256][256] cfg->dtype
 *   probs [batch][1000] fp32, mean of the ten views' softmax outputs */
int alexnet_forward_tenview(const alexnet_cfg* cfg, const void* const params[16], const void* src,
                            float* probs, void* ws, size_t ws_bytes, void* stream);

/* One training step (fermi.ai TRAIN_STEP; paper-graph-ui "Dropout" and
 * "Training Procedure Details"): forward with dropout masks drawn from
 * Philox4x32-10 keyed by (seed, step) (see alexnet_dropout_mask), the mean
 * cross-entropy of the softmax w.r.t. `labels`, backpropagation through all
 * eight layers, then for each of the 16 parameter tensors
 *     v <- momentum*v - weight_decay*lr*w - lr*g ;  w <- w + v
 * on the fp32 master weights, and the working copies refreshed from the new
 * master (round to nearest even for bf16).
 *   master[16]   fp32, in/out          momentum[16] fp32, in/out
 *   work[16]     cfg->dtype, in (used by forward/backward), out (refreshed)
 *   x            [batch][3][227][227] cfg->dtype
 *   labels       [batch] int32 in [0, 1000); out-of-range labels give an
 *                undefined loss and gradient but never an out-of-bounds access
 *   loss         one fp32 (device), the batch-mean cross-entropy
 *   probs        optional [batch][1000] fp32 softmax output (may be null)
 * Each tensor is updated as soon as its gradient is complete: the three FC
 * weight tensors inside the GEMM that forms their gradient (after that layer's
 * data gradient has read the old working weights), the conv weights as their
 * split-K gradient is reduced (the data gradients read a copy of the old
 * weights made at the start of the step), the biases with their gradients.
 * Every gradient is therefore that of the pre-step weights.  The conv weight
 * gradients and all bias gradients stay in the workspace (taps gw1..gw5,
 * gb1..gb8) until the next call; the FC weight gradients are never stored and
 * gw6..gw8 do not exist (alexnet_tap returns ALEXNET_E_ARG). */
int alexnet_train_step(const alexnet_cfg* cfg, float* const master[16], float* const momentum[16],
                       void* const work[16], const void* x, const int32_t* labels, float lr,
                       float momentum_coef, float weight_decay, uint64_t seed, uint64_t step,
                       float* loss, float* probs, void* ws, size_t ws_bytes, void* stream);

/* Training-time data augmentation (ImageNet Classification with Deep
 * Convolutional Neural Networks, section 4.1, both forms), fed straight into
 * the layer-1 input staging of a training step.  Image n of the batch is
 *   x[n][c][y][x'] = src[n][c][y0 + y][x0 + (flip ? 226 - x' : x')]
 *                    + sum_i eigvec[c][i] * alpha[n][i] * eigval[i]
 * for y, x' in [0, 227): a 227 x 227 patch of source n, mirrored left-right
 * when flip != 0, plus the colour shift along the principal components of the
 * RGB values (one draw alpha[n][0..2] per image, N(0, 0.1) on the pages).
 * The shift is formed in fp32 as eigvec[c][0]*(alpha0*eigval0), then two
 * fused multiply-adds for i = 1, 2; the pixel plus shift is rounded once to
 * cfg->dtype (round to nearest even for bf16).  The random draws are the
 * caller's: crop offsets, flips and alpha are inputs.
 *   crop    device int32 [batch][3]: y0, x0, flip.  Offsets outside
 *           [0, src_h - 227] x [0, src_w - 227] are clamped into it (never an
 *           out-of-bounds read).
 *   alpha   device fp32 [batch][3]
 *   eigval  device fp32 [3]; eigvec device fp32 [3][3], row c = colour
 *           channel, column i = component i (as alexnet_rgb_pca writes them) */
typedef struct {
  const int32_t* crop;
  const float* alpha;
  const float* eigval;
  const float* eigvec;
} alexnet_augment;

/* x [batch][3][227][227] cfg->dtype (written) = the augmented patches of
 * src [batch][3][src_h][src_w] (cfg->dtype), 227 <= src_h, src_w <= 8192.
 * The same values alexnet_train_step_augmented stages for layer 1. */
int alexnet_augment_images(const alexnet_cfg* cfg, const void* src, int32_t src_h, int32_t src_w,
                           const alexnet_augment* aug, void* x, void* stream);

/* alexnet_train_step on the augmented patches of src [batch][3][src_h][src_w]
 * (cfg->dtype): the patches are read from the sources by the layer-1 input
 * staging and never stored.  Same workspace (ALEXNET_MODE_TRAIN), outputs and
 * results as alexnet_train_step on the output of alexnet_augment_images. */
int alexnet_train_step_augmented(const alexnet_cfg* cfg, float* const master[16],
                                 float* const momentum[16], void* const work[16], const void* src,
                                 int32_t src_h, int32_t src_w, const alexnet_augment* aug,
                                 const int32_t* labels, float lr, float momentum_coef,
                                 float weight_decay, uint64_t seed, uint64_t step, float* loss,
                                 float* probs, void* ws, size_t ws_bytes, void* stream);

/* Principal components of the RGB values of all pixels of n images
 * [n][3][h][w] (cfg->dtype; only cfg->dtype is read), the statistic the
 * colour augmentation uses (section 4.1: the 3 x 3 covariance of the RGB
 * pixel values, its eigenvectors p_i and eigenvalues lambda_i).  The
 * covariance divides by the pixel count n*h*w; moments accumulate in fp64
 * (exact for bf16 inputs), and cyclic Jacobi rotations diagonalise it in fp64.
 *   eigval  device fp32 [3] (written), descending
 *   eigvec  device fp32 [3][3] (written), column i the unit eigenvector of
 *           eigval[i], signed so that its largest-magnitude entry is positive
 *   ws      device scratch of alexnet_rgb_pca_workspace_bytes(), 256-aligned
 * Equal eigenvalues leave their eigenvectors' directions to the rotation
 * sequence; the pages' use of them is unaffected. */
size_t alexnet_rgb_pca_workspace_bytes(void);
int alexnet_rgb_pca(const alexnet_cfg* cfg, const void* images, int32_t n, int32_t h, int32_t w,
                    float* eigval, float* eigvec, void* ws, size_t ws_bytes, void* stream);

/* work[i] <- cfg->dtype copy of master[i] (round to nearest even), all 16
 * tensors.  For fp32 work tensors this is a copy. */
int alexnet_cast_weights(const alexnet_cfg* cfg, float* const master[16], void* const work[16],
                         void* stream);

/* The dropout keep-mask used by alexnet_train_step for layer `layer`
 * (0 = fc6, 1 = fc7) at `step`: mask[r][c] = 1 keeps unit c of row r, 0 drops
 * it.  Element e = r*cols + c takes word (e mod 4) of
 * Philox4x32-10(counter = (e/4, layer, step mod 2^32, step / 2^32),
 *              key = (seed mod 2^32, seed / 2^32))
 * and is dropped iff that word < floor(p * 2^32).  cols must be a multiple
 * of 4.  mask: device [rows][cols] uint8 (written). */
int alexnet_dropout_mask(uint64_t seed, uint64_t step, int32_t layer, int32_t rows, int32_t cols,
                         float p, uint8_t* mask, void* stream);

/* Kernel timing (diagnostics).  The *_timed variants behave exactly like
 * the plain calls and additionally record caller-created HIP events
 * (hipEvent_t handles passed as void*) on `stream` immediately before and
 * after the launch of the named kernel; for GEMM layers that is the product
 * kernel alone (the MFMA GEMM, or for an FC layer of at most 4 rows the row
 * kernel), not its split-K reduction.  (The timed training calls run with no
 * side stream; see alexnet_train_step_ex for timers beside one.)  The exception to
 * the first rule is a convolution split
 * over k because the batch is too small to fill the chip (never at batch
 * 128): its events also cover the reduction, which applies its epilogue.  A
 * kernel the call does not launch records nothing.  timers may be NULL when
 * n_timers is 0. */
typedef enum {
  ALEXNET_KT_S2D = 1,          /* layer-1 input staging (4x4 pixel blocks) and all
                                  weight re-layouts of the call, one launch      */
  ALEXNET_KT_CONV1_FWD, ALEXNET_KT_CONV2_FWD, ALEXNET_KT_CONV3_FWD, ALEXNET_KT_CONV4_FWD,
  ALEXNET_KT_CONV5_FWD,
  ALEXNET_KT_LRNPOOL1_FWD,     /* LRN1 + pool1 (one fused kernel)                */
  ALEXNET_KT_LRNPOOL2_FWD,     /* LRN2 + pool2                                   */
  ALEXNET_KT_POOL5_FWD,
  ALEXNET_KT_FC6_FWD, ALEXNET_KT_FC7_FWD, ALEXNET_KT_FC8_FWD,
  ALEXNET_KT_FC8_DGRAD, ALEXNET_KT_FC7_DGRAD, ALEXNET_KT_FC6_DGRAD,
  ALEXNET_KT_FC8_WGRAD, ALEXNET_KT_FC7_WGRAD, ALEXNET_KT_FC6_WGRAD,
  ALEXNET_KT_POOL5_BWD,
  ALEXNET_KT_CONV5_WGRAD, ALEXNET_KT_CONV4_WGRAD, ALEXNET_KT_CONV3_WGRAD, ALEXNET_KT_CONV2_WGRAD,
  ALEXNET_KT_CONV1_WGRAD,
  ALEXNET_KT_CONV5_DGRAD, ALEXNET_KT_CONV4_DGRAD, ALEXNET_KT_CONV3_DGRAD, ALEXNET_KT_CONV2_DGRAD,
  ALEXNET_KT_POOLLRN2_BWD,     /* pool2, LRN2 and ReLU2 backward (one kernel)    */
  ALEXNET_KT_POOLLRN1_BWD,     /* pool1, LRN1 and ReLU1 backward                 */
  ALEXNET_KT_BIAS,             /* bias gradients of layers 3-8 + their SGD (two
                                  launches)                                      */
  ALEXNET_KT_RGB_PCA,          /* alexnet_rgb_pca: moments + eigen-decomposition */
  ALEXNET_KT_BIAS12,           /* bias gradients of layers 1 and 2 from their row
                                  sums + their SGD, and the batch-mean loss (two
                                  launches)                                      */
  ALEXNET_KT_COUNT
} alexnet_kernel;

typedef struct {
  int32_t kernel;  /* alexnet_kernel */
  void* start;     /* hipEvent_t recorded before the launch */
  void* stop;      /* hipEvent_t recorded after the launch  */
} alexnet_timer;

int alexnet_forward_timed(const alexnet_cfg* cfg, const void* const params[16], const void* x,
                          float* probs, void* ws, size_t ws_bytes, void* stream,
                          const alexnet_timer* timers, int32_t n_timers);
int alexnet_train_step_timed(const alexnet_cfg* cfg, float* const master[16],
                             float* const momentum[16], void* const work[16], const void* x,
                             const int32_t* labels, float lr, float momentum_coef,
                             float weight_decay, uint64_t seed, uint64_t step, float* loss,
                             float* probs, void* ws, size_t ws_bytes, void* stream,
                             const alexnet_timer* timers, int32_t n_timers);
int alexnet_train_step_augmented_timed(const alexnet_cfg* cfg, float* const master[16],
                                       float* const momentum[16], void* const work[16],
                                       const void* src, int32_t src_h, int32_t src_w,
                                       const alexnet_augment* aug, const int32_t* labels, float lr,
                                       float momentum_coef, float weight_decay, uint64_t seed,
                                       uint64_t step, float* loss, float* probs, void* ws,
                                       size_t ws_bytes, void* stream, const alexnet_timer* timers,
                                       int32_t n_timers);
int alexnet_rgb_pca_timed(const alexnet_cfg* cfg, const void* images, int32_t n, int32_t h,
                          int32_t w, float* eigval, float* eigvec, void* ws, size_t ws_bytes,
                          void* stream, const alexnet_timer* timers, int32_t n_timers);

/* The training step with every option (all other training entry points are
 * this call with some options fixed):
 *   aug          NULL: x is images [batch][3][227][227] and src_h, src_w are
 *                ignored; else x is sources [batch][3][src_h][src_w] and the
 *                call is alexnet_train_step_augmented.
 *   ex           may be NULL (no side stream, no timers).
 *   ex->side_stream  a caller-owned hipStream_t other than `stream`, or NULL.
 *                Given one, the layers' weight gradients with their SGD
 *                updates run on it, each forked from `stream` (event record +
 *                stream wait) once the gradient w.r.t. that layer's output is
 *                complete, while `stream` carries on with the data gradients;
 *                the side stream is joined back to `stream` before the call
 *                returns.  Results are bit-identical to the serial order: no
 *                kernel of either chain reads what the other writes, and every
 *                reduction runs in a fixed order.  The step stays serial when
 *                a conv data gradient splits over k (small batches share the
 *                split-K scratch with the weight gradients).  NULL:
 *                everything runs on `stream` in order.
 *   ex->events   ALEXNET_SIDE_EVENTS caller-created hipEvent_t handles (timing
 *                may be disabled), all non-null when side_stream is set;
 *                recorded and waited on by every call, never created or
 *                destroyed by the library.  Reusing them across calls is safe:
 *                a stream wait binds to the record enqueued before it.  Two
 *                calls in flight at once need distinct sets.
 *   ex->timers, ex->n_timers  as for alexnet_train_step_timed; timers do not
 *                change the order above.  A timed kernel that runs on the
 *                side stream has its events recorded there, and the time of
 *                any kernel then includes the GPU it shares with the kernels
 *                of the other stream (for isolated times: no side stream).
 * Returns ALEXNET_E_ARG if side_stream == stream, ALEXNET_E_NULL if an event
 * is missing. */
#define ALEXNET_SIDE_EVENTS 10
typedef struct {
  void* side_stream;
  void* events[ALEXNET_SIDE_EVENTS];
  const alexnet_timer* timers;
  int32_t n_timers;
} alexnet_exec;

int alexnet_train_step_ex(const alexnet_cfg* cfg, float* const master[16], float* const momentum[16],
                          void* const work[16], const void* x, const alexnet_augment* aug, int32_t src_h,
                          int32_t src_w, const int32_t* labels, float lr, float momentum_coef,
                          float weight_decay, uint64_t seed, uint64_t step, float* loss, float* probs, void* ws,
                          size_t ws_bytes, void* stream, const alexnet_exec* ex);

/* Events for ex->events and for kernel timers, created without the
 * system-scope memory fence that a default HIP event carries: a default event
 * writes the GPU caches back for the host's sake when it completes, which
 * idles the GPU for some microseconds at every record and, for a timer,
 * counts that write-back in the timed kernel.  Kernels of one device see each
 * other's results across streams without that fence; the host does not, so
 * these events order device work (stream waits, timing) and do not make
 * results visible to the host (synchronize the stream for that).
 *   timing != 0: the event can be timed (alexnet_event_elapsed_ms); else
 *   timing is disabled.  The caller owns the event and destroys it with
 *   alexnet_event_destroy.  Host only; creates a HIP event on the current
 *   device.  Returns ALEXNET_E_NULL for a null pointer, ALEXNET_E_HIP if
 *   the HIP call fails. */
int alexnet_event_create(int32_t timing, void** event);
int alexnet_event_destroy(void* event);
/* Milliseconds from `start` to `stop`, two completed timing events. */
int alexnet_event_elapsed_ms(void* start, void* stop, float* ms);

/* Test and diagnostic access to the tensors a call leaves in its workspace.
 * Host only.  For tap `tap_id` of a call in `mode` with `cfg`, returns its
 * byte offset into the workspace, its shape (unused trailing dims = 1), its
 * element type (alexnet_dtype) and its layout: 0 = NHWC activation
 * [N][H][W][C], 1 = row-major matrix / vector, 2 = OIHW or [out][in] weight
 * gradient (fp32).  Returns ALEXNET_E_ARG for a tap the mode does not have. */
int alexnet_tap(const alexnet_cfg* cfg, int mode, int tap_id, size_t* offset, int64_t shape[4],
                int* dtype, int* layout);
int alexnet_tap_count(void);
const char* alexnet_tap_name(int tap_id); /* NULL if out of range */

const char* alexnet_status_string(int status);

#ifdef __cplusplus
}
#endif
#endif /* ALEXNET_H */
