// la_chunk_linear.hip -- chunked forward of normalized and gated linear attention.
#include "la_internal.hpp"
namespace la {
hipError_t launch_chunk_linear(const ChunkArgs &) { return hipErrorNotSupported; }
}  // namespace la
