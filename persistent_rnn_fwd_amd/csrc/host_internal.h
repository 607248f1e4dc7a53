// Host-side pieces of the library shared between its translation units (not
// part of the C ABI).
#pragma once

#include <stddef.h>
#include <stdint.h>

#include "prnn.h"

namespace prnn {

// What a call needs to know about its device, found once per device.
struct DeviceFacts {
  int num_cu = 0;
  size_t lds_per_block = 0;
  bool placement_round_robin = false;  // workgroup i of a cooperative launch runs on XCD (i + c) % 8
  bool plain_placement = false;        // ... and of a plain launch (then launched plainly)
};

// Words of exchange memory a team-layout call of width N needs: [8 XCD][2 slots][Npad].
inline size_t team_ring_words(int N) { return 16u * (size_t)((N + 3) & ~3); }

// One dense forward call (the operation of prnn_forward_dense, default
// options) in the team layout, on exchange memory and a status word the
// caller provides: `ring` holds at least team_ring_words(N) words and is
// reset by the call, `status` (one device word) is cleared by the call and
// set to a nonzero value if the run fails.  Argument checks and errors as
// prnn_forward_dense; shapes the team layout cannot take return
// NOT_SUPPORTED.  Allocates nothing.
prnnStatus_t forward_dense_on(const DeviceFacts& dev, uint32_t* ring, uint32_t* status, int N, int B, int T,
                              prnnDataType_t w_type, const void* W, const float* X, const float* h0, float* H,
                              hipStream_t stream);

}  // namespace prnn
