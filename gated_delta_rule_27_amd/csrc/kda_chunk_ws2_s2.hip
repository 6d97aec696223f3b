// kda_chunk_ws2_s2.hip -- the half-head prefill with outputs (split 2: 4
// state waves, 64 value columns per workgroup) of the pipelined bf16
// kernel (kda_chunk_ws2_impl.h), in a translation unit of its own so that
// it can be built with LLVM's iterative ILP machine scheduler
// (-amdgpu-sched-strategy=iterative-ilp, set in build.py).  On MI355X that
// schedule of its role loops takes the 4096-token, 96-head prefill from
// 233 us to 220 us with the same results bit for bit.  The other variants
// stay with the default scheduler: under the iterative one the whole-head
// kernel spills to scratch and the paired summary passes run 15% slower.
#include "kda_chunk_ws2_impl.h"

namespace kda {

hipError_t launch_chunk_ws2_split2(const ChunkArgs& a, hipStream_t stream) {
    return launch_ws2_t<4, false>(a, stream);
}

}  // namespace kda
