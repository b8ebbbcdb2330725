// la_chunk_gdr.hip -- chunked forward of the gated delta rule.
#include "la_internal.hpp"
namespace la {
hipError_t launch_chunk_linear(const ChunkArgs &a);
hipError_t launch_chunk_gdr(const ChunkArgs &) { return hipErrorNotSupported; }
size_t chunk_workspace_bytes(const ChunkArgs &) { return 0; }
hipError_t launch_chunk(const ChunkArgs &a) {
    return a.variant == LA_GATED_DELTA ? launch_chunk_gdr(a) : launch_chunk_linear(a);
}
}  // namespace la
