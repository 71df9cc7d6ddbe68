// Multi-row segments (prompt chunks, speculative drafts) on bf16 MFMA tiles.
#include "pkv_device.h"
#include "pkv_internal.h"

namespace pkv {

bool chunk_supported(int32_t dtype, int32_t head_dim, int32_t group) {
  (void)dtype;
  (void)head_dim;
  (void)group;
  return false;
}

int launch_chunk(const AttendArgs &a, int32_t head_dim, int32_t max_query_len, int32_t max_context_len,
                 hipStream_t stream) {
  (void)a;
  (void)head_dim;
  (void)max_query_len;
  (void)max_context_len;
  (void)stream;
  return PKV_ERR_UNSUPPORTED;
}

}  // namespace pkv
