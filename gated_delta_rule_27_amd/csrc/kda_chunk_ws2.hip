// kda_chunk_ws2.hip -- launches of the pipelined bf16 prefill kernel
// (kda_chunk_ws2_impl.h) and the dispatch over its variants; the half-head
// prefill with outputs is instantiated in kda_chunk_ws2_s2.hip.
#include "kda_chunk_ws2_impl.h"

namespace kda {

bool chunk_ws2_supports(const ChunkArgs& a, int split) {
    if (a.flags & kChunkDualBM) return split == 2 && !a.snap.snap && (a.flags & kChunkNoOutput);
    return split == 1 || split == 2;
}

hipError_t launch_chunk_ws2(const ChunkArgs& a, int split, hipStream_t stream) {
    if (!chunk_ws2_supports(a, split)) return hipErrorInvalidValue;
    if (a.flags & kChunkDualBM) return launch_ws2_t<4, true, true>(a, stream);
    if (a.flags & kChunkNoOutput)
        return split == 1 ? launch_ws2_t<8, true>(a, stream) : launch_ws2_t<4, true>(a, stream);
    return split == 1 ? launch_ws2_t<8, false>(a, stream) : launch_chunk_ws2_split2(a, stream);
}

}  // namespace kda
