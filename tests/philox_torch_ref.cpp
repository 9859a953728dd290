// Test-only reference for the Philox4x32-10 pin: a thin C wrapper around
// PyTorch's source-level Philox engine (ATen/core/PhiloxRNGEngine.h, written
// from Salmon et al., "Parallel Random Numbers: As Easy as 1, 2, 3", SC'11).
// It is an implementation independent of the oracle's and of the HIP path's.
// The engine's counter is (offset lo, offset hi, subsequence lo, subsequence
// hi) and its key is (seed lo, seed hi); the first four 32-bit draws after
// construction are the four output words of the block at that counter.
#include <ATen/core/PhiloxRNGEngine.h>
#include <cstdint>

extern "C" void ref_philox_block(uint64_t seed, uint64_t subsequence, uint64_t offset,
                                 uint32_t out[4]) {
  at::philox_engine eng(seed, subsequence, offset);
  for (int i = 0; i < 4; ++i) out[i] = eng();
}
