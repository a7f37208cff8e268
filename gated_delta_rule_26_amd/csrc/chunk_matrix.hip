// Matrix-core (bf16 MFMA) chunked path: not built yet.  The API reports it as
// unavailable and routes every call to the vector path.
#include "gdr_internal.h"

namespace gdr {

size_t chunk_matrix_workspace_bytes(int, int, int, int, int, bool) { return 0; }

hipError_t launch_chunk_matrix(const ChunkArgs &, int) { return hipErrorNotSupported; }

}  // namespace gdr
